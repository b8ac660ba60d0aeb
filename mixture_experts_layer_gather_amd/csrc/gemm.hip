// Grouped expert GEMMs on gfx950 matrix cores (MFMA), forward and backward.
//
// Many small expert GEMMs become one launch (Megatron Core MoE summary,
// section 2.4, "Grouped GEMM"), which matters most for fine-grained MoE whose
// per-expert GEMMs are tall and skinny (Piper summary, section 1; Megatron
// Core summary, section 1, the compute-efficiency wall). Expert loads may be
// skewed (Hybrid-EP article, hot and cold experts), so work is split into
// tiles, not experts: every workgroup owns one output tile, and the
// tile -> (expert, row tile, column tile) map is computed on the device from
// the expert offsets (Megatron Core summary, section 2.4, device-initiated
// kernels): nothing about the routing is ever read on the host.
//
// One template covers the six GEMMs of a SwiGLU expert:
//   forward   GU = X W1^T (+ SwiGLU epilogue)   A [M,K] K-major, B [N,K] K-major
//             O  = H W2^T                        A K-major, B K-major
//   dgrad     dH = dO W2 (+ SwiGLU backward)     A K-major, B [K,N] N-major
//             dX = dGU W1                        A K-major, B N-major
//   wgrad     dW2 = dO^T H, dW1 = dGU^T X        A [K,M], B [K,N]; K = the
//                                                expert's rows (ragged)
// Tiles are staged through LDS (double buffered, one barrier per K step) in
// K-contiguous rows so that every MFMA operand is one 16-byte LDS read;
// operands stored the other way round are transposed on their way into LDS.
// Workgroup ids are remapped so that each XCD (8 per chip, one L2 each) works
// through a contiguous range of tiles that share weights and rows.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

enum { G_ROWS = 0, G_KSPLIT = 1 };
enum { EPI_STORE = 0, EPI_SWIGLU = 1, EPI_DSWIGLU = 2 };

template <typename T> struct Mfma;
template <> struct Mfma<bf16_t> {
  static constexpr int KP = 8;   // elements per lane per instruction
  static constexpr int MK = 32;  // K per instruction
  typedef bf16x8_t frag;
  static __device__ __forceinline__ frag load(const bf16_t* p) {
    return __builtin_bit_cast(frag, *reinterpret_cast<const u32x4*>(p));
  }
  static __device__ __forceinline__ f32x4_t mma(frag a, frag b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mfma<float> {
  static constexpr int KP = 1;
  static constexpr int MK = 4;
  typedef float frag;
  static __device__ __forceinline__ frag load(const float* p) { return *p; }
  static __device__ __forceinline__ f32x4_t mma(frag a, frag b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

struct GemmArgs {
  const void* A;
  int64_t lda;
  const void* B;
  int64_t ldb;
  int64_t b_gstride;  // elements between consecutive groups' B (ROWS)
  void* C;
  int64_t ldc;
  int64_t c_gstride;  // elements between consecutive groups' C (KSPLIT)
  const int32_t* offsets;
  int G;
  int M, N, K;        // ROWS: N, K used; KSPLIT: M, N used
  int f;              // SwiGLU half width
  void* aux0;         // SWIGLU: GU out [rows,2f]; DSWIGLU: GU in
  void* aux1;         // SWIGLU: H out [rows,f]
  int tiles_n;
  int tiles_m;        // KSPLIT
};

// Bijective remap of workgroup ids: consecutive ids are spread over the 8
// XCDs round robin, so give XCD x the x-th contiguous slice of tiles.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  const int q = nblocks / 8, r = nblocks % 8;
  const int x = bid % 8, i = bid / 8;
  return x * q + min(x, r) + i;
}

// Exclusive scan of per-group row-tile counts; returns the tile's group in
// s_info[0], its row-tile count in s_info[1] and the first tile of the group
// in s_info[2], or s_info[0] = -1 when the tile is past the end.
template <int BM>
__device__ void find_group(const int32_t* __restrict__ offsets, int G, int tiles_n, int tile,
                           int* s_scan, int* s_info) {
  const int tid = threadIdx.x;
  constexpr int PER = 4;  // groups per thread (G <= 1024)
  int cnt[PER], local = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int g = tid * PER + i;
    int c = 0;
    if (g < G) {
      const int m = offsets[g + 1] - offsets[g];
      c = (m + BM - 1) / BM;
    }
    cnt[i] = c;
    local += c;
  }
  // inclusive scan of `local` across the 256 threads
  int v = local;
  const int lane = lane_id();
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o, kWave);
    if (lane >= o) v += u;
  }
  const int wave = tid / kWave;
  if (lane == 63) s_scan[wave] = v;
  if (tid == 0) s_info[0] = -1;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += s_scan[w];
  int start = before + v - local;  // exclusive prefix (in row tiles)
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int g = tid * PER + i;
    if (g < G && cnt[i] > 0) {
      const int t0 = start * tiles_n, t1 = (start + cnt[i]) * tiles_n;
      if (tile >= t0 && tile < t1) {
        s_info[0] = g;
        s_info[1] = cnt[i];
        s_info[2] = t0;
      }
    }
    start += cnt[i];
  }
  __syncthreads();
}

// LDS tiles hold ROWS x BK elements per operand, K-contiguous, without
// padding. The 16-byte chunks of each row are XOR-swizzled with the row so
// that both the MFMA fragment reads (16 consecutive rows, one chunk each) and
// the transposed stores (rows 8 apart) spread over all banks.
template <typename T, int BK>
__device__ __forceinline__ int lds_off(int row, int k) {
  constexpr int VEC = 16 / sizeof(T);
  constexpr int NCH = BK / VEC;
  const int sw = (row ^ (row >> 3)) & (NCH - 1);
  return row * BK + (((k / VEC) ^ sw) * VEC) + (k % VEC);
}

// 4 K-rows x VEC columns (four 16-byte registers) -> VEC LDS rows of 4
// K-values each.
template <typename T, int BK>
__device__ __forceinline__ void store_transposed(const u32x4* r, T* dst, int c0, int k4) {
  const uint32_t w[4][4] = {{r[0][0], r[0][1], r[0][2], r[0][3]}, {r[1][0], r[1][1], r[1][2], r[1][3]},
                            {r[2][0], r[2][1], r[2][2], r[2][3]}, {r[3][0], r[3][1], r[3][2], r[3][3]}};
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const u32x2 ev = {(w[0][p] & 0xffffu) | (w[1][p] << 16), (w[2][p] & 0xffffu) | (w[3][p] << 16)};
      const u32x2 od = {(w[0][p] >> 16) | (w[1][p] & 0xffff0000u), (w[2][p] >> 16) | (w[3][p] & 0xffff0000u)};
      *reinterpret_cast<u32x2*>(dst + lds_off<T, BK>(c0 + 2 * p, k4)) = ev;
      *reinterpret_cast<u32x2*>(dst + lds_off<T, BK>(c0 + 2 * p + 1, k4)) = od;
    }
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const u32x4 v = {w[0][c], w[1][c], w[2][c], w[3][c]};
      *reinterpret_cast<u32x4*>(dst + lds_off<T, BK>(c0 + c, k4)) = v;
    }
  }
}

// Per-thread plan for moving one operand tile (ROWS x BK, stored K-major in
// LDS) from global memory: the thread's source pointers are fixed for the
// whole K loop and advance by k0 elements (K-major source) or k0 rows
// (K-strided source).
//   K-major source:   N16 chunks of 16 bytes, chunk i = (row r_i, k-chunk c_i)
//   K-strided source: NT blocks of 4 K-rows x VEC columns
template <typename T, bool KMAJ, int ROWS, int BK>
struct OperandPlan {
  static constexpr int VEC = 16 / sizeof(T);
  static constexpr int N16 = ROWS * BK / VEC / 256;
  static constexpr int NT = BK * ROWS / (4 * VEC) / 256;
  static constexpr int NREG = KMAJ ? N16 : 4 * NT;
  static constexpr int NPTR = KMAJ ? N16 : NT;
  static_assert(NPTR >= 1, "tile too small for 256 threads");
  const T* ptr[NPTR];
  int lrow[NPTR];  // LDS row (K-major) or first LDS row (K-strided)
  int lk[NPTR];    // LDS k offset
  int kr[NPTR];    // K-strided: first K-row of the block (for masking)
  bool ok[NPTR];   // K-major: row is valid
};

template <typename T, int BM, int BN, int BK>
struct Smem {
  T A[2][BM * BK];
  T B[2][BN * BK];
};

template <typename T, typename TC, bool A_KMAJ, bool B_KMAJ, int MODE, int EPI, int BM, int BN,
          int BK, int WM, int WN>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs g) {
  using MF = Mfma<T>;
  using SM = Smem<T, BM, BN, BK>;
  constexpr int VEC = 16 / sizeof(T);
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 16, FN = WTN / 16;
  using PA = OperandPlan<T, A_KMAJ, BM, BK>;
  using PB = OperandPlan<T, B_KMAJ, BN, BK>;
  static_assert(WM * WN == 4, "four waves");
  static_assert(EPI != EPI_SWIGLU || FN % 2 == 0, "SwiGLU pairs column fragments");

  __shared__ __attribute__((aligned(16))) SM sm;
  __shared__ int s_scan[4];
  __shared__ int s_info[3];

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid / kWave;
  const int wm = wave / WN, wn = wave % WN;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);

  int grp, mt, nt;
  int row0;           // first A row (ROWS) of the tile
  int mrows;          // valid rows in the tile (ROWS)
  int kbase, kcount;  // contraction range
  if (MODE == G_ROWS) {
    find_group<BM>(g.offsets, g.G, g.tiles_n, tile, s_scan, s_info);
    grp = s_info[0];
    if (grp < 0) return;
    const int cnt = s_info[1];
    const int local = tile - s_info[2];
    nt = local / cnt;
    mt = local % cnt;
    row0 = g.offsets[grp] + mt * BM;
    mrows = min(BM, g.offsets[grp + 1] - row0);
    kbase = 0;
    kcount = g.K;
  } else {
    const int per = g.tiles_m * g.tiles_n;
    grp = tile / per;
    if (grp >= g.G) return;
    const int rem = tile % per;
    mt = rem / g.tiles_n;
    nt = rem % g.tiles_n;
    row0 = 0;
    mrows = BM;
    kbase = g.offsets[grp];
    kcount = g.offsets[grp + 1] - kbase;
  }

  const T* __restrict__ Ab = reinterpret_cast<const T*>(g.A);
  const T* __restrict__ Bb = reinterpret_cast<const T*>(g.B);
  if (MODE == G_ROWS) Bb += int64_t(grp) * g.b_gstride;
  const int m0 = mt * BM;  // KSPLIT: output row block
  const int n0 = nt * BN;

  // ---- per-thread load plans
  PA pa;
  PB pb;
  if constexpr (A_KMAJ) {
#pragma unroll
    for (int i = 0; i < PA::NPTR; ++i) {
      const int q = tid + i * 256;
      const int r = q / (BK / VEC), kc = q % (BK / VEC);
      pa.lrow[i] = r;
      pa.lk[i] = kc * VEC;
      pa.ok[i] = r < mrows;
      pa.ptr[i] = Ab + int64_t(row0 + (r < mrows ? r : 0)) * g.lda + kc * VEC;
    }
  } else {
#pragma unroll
    for (int i = 0; i < PA::NPTR; ++i) {
      const int q = tid + i * 256;
      const int kq = q / (BM / VEC), mc = q % (BM / VEC);
      pa.lrow[i] = mc * VEC;
      pa.lk[i] = 4 * kq;
      pa.kr[i] = 4 * kq;
      pa.ptr[i] = Ab + int64_t(kbase + 4 * kq) * g.lda + m0 + mc * VEC;
    }
  }
  if constexpr (B_KMAJ) {
#pragma unroll
    for (int i = 0; i < PB::NPTR; ++i) {
      const int q = tid + i * 256;
      const int r = q / (BK / VEC), kc = q % (BK / VEC);
      int grow = n0 + r;
      if (EPI == EPI_SWIGLU) {
        // gate and up rows of the same output columns side by side within
        // each wave's column range
        const int w = r / WTN, within = r % WTN;
        const int half = within / (WTN / 2), j = within % (WTN / 2);
        grow = half * g.f + nt * (BN / 2) + w * (WTN / 2) + j;
      }
      pb.lrow[i] = r;
      pb.lk[i] = kc * VEC;
      pb.ok[i] = true;
      pb.ptr[i] = Bb + int64_t(grow) * g.ldb + kc * VEC;
    }
  } else {
#pragma unroll
    for (int i = 0; i < PB::NPTR; ++i) {
      const int q = tid + i * 256;
      const int kq = q / (BN / VEC), nc = q % (BN / VEC);
      pb.lrow[i] = nc * VEC;
      pb.lk[i] = 4 * kq;
      pb.kr[i] = 4 * kq;
      pb.ptr[i] = Bb + int64_t(kbase + 4 * kq) * g.ldb + n0 + nc * VEC;
    }
  }

  u32x4 ra[PA::NREG], rb[PB::NREG];
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  // global -> registers for the K step starting at k0
#define MOE_GLOAD(k0)                                                                           \
  do {                                                                                          \
    if constexpr (A_KMAJ) {                                                                     \
      _Pragma("unroll") for (int i = 0; i < PA::NPTR; ++i) {                                    \
        ra[i] = pa.ok[i] ? *reinterpret_cast<const u32x4*>(pa.ptr[i] + (k0)) : zero4; \
      }                                                                                         \
    } else {                                                                                    \
      _Pragma("unroll") for (int i = 0; i < PA::NPTR; ++i) {                                    \
        _Pragma("unroll") for (int j = 0; j < 4; ++j) {                                         \
          const bool v = (k0) + pa.kr[i] + j < kcount;                                          \
          ra[4 * i + j] = v ? *reinterpret_cast<const u32x4*>(pa.ptr[i] + int64_t((k0) + j) * g.lda) \
                            : zero4;                                           \
        }                                                                                       \
      }                                                                                         \
    }                                                                                           \
    if constexpr (B_KMAJ) {                                                                     \
      _Pragma("unroll") for (int i = 0; i < PB::NPTR; ++i) {                                    \
        rb[i] = *reinterpret_cast<const u32x4*>(pb.ptr[i] + (k0));                              \
      }                                                                                         \
    } else {                                                                                    \
      _Pragma("unroll") for (int i = 0; i < PB::NPTR; ++i) {                                    \
        _Pragma("unroll") for (int j = 0; j < 4; ++j) {                                         \
          const bool v = MODE == G_ROWS || (k0) + pb.kr[i] + j < kcount;                        \
          rb[4 * i + j] = v ? *reinterpret_cast<const u32x4*>(pb.ptr[i] + int64_t((k0) + j) * g.ldb) \
                            : zero4;                                           \
        }                                                                                       \
      }                                                                                         \
    }                                                                                           \
  } while (0)
  // registers -> LDS buffer `buf`
#define MOE_LSTORE(buf)                                                                         \
  do {                                                                                          \
    if constexpr (A_KMAJ) {                                                                     \
      _Pragma("unroll") for (int i = 0; i < PA::NPTR; ++i)                                      \
        *reinterpret_cast<u32x4*>(&sm.A[buf][lds_off<T, BK>(pa.lrow[i], pa.lk[i])]) = ra[i];    \
    } else {                                                                                    \
      _Pragma("unroll") for (int i = 0; i < PA::NPTR; ++i)                                      \
        store_transposed<T, BK>(&ra[4 * i], sm.A[buf], pa.lrow[i], pa.lk[i]);                   \
    }                                                                                           \
    if constexpr (B_KMAJ) {                                                                     \
      _Pragma("unroll") for (int i = 0; i < PB::NPTR; ++i)                                      \
        *reinterpret_cast<u32x4*>(&sm.B[buf][lds_off<T, BK>(pb.lrow[i], pb.lk[i])]) = rb[i];    \
    } else {                                                                                    \
      _Pragma("unroll") for (int i = 0; i < PB::NPTR; ++i)                                      \
        store_transposed<T, BK>(&rb[4 * i], sm.B[buf], pb.lrow[i], pb.lk[i]);                   \
    }                                                                                           \
  } while (0)

  f32x4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  const int nk = (kcount + BK - 1) / BK;
  if (nk > 0) {
    MOE_GLOAD(0);
    MOE_LSTORE(0);
    __syncthreads();
  }
  for (int s = 0; s < nk; ++s) {
    const int buf = s & 1;
    if (s + 1 < nk) MOE_GLOAD((s + 1) * BK);
#pragma unroll
    for (int kk = 0; kk < BK / MF::MK; ++kk) {
      const int kofs = kk * MF::MK + (lane / 16) * MF::KP;
      typename MF::frag af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = MF::load(&sm.A[buf][lds_off<T, BK>(wm * WTM + i * 16 + (lane % 16), kofs)]);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bfr[j] = MF::load(&sm.B[buf][lds_off<T, BK>(wn * WTN + j * 16 + (lane % 16), kofs)]);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = MF::mma(af[i], bfr[j], acc[i][j]);
    }
    if (s + 1 < nk) MOE_LSTORE(buf ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds rows 4*(lane/16)+r, column lane%16 of each 16x16
  const int lr = 4 * (lane / 16), lc = lane % 16;
  if (EPI == EPI_STORE) {
    TC* Cb = reinterpret_cast<TC*>(g.C);
    if (MODE == G_KSPLIT) Cb += int64_t(grp) * g.c_gstride;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int rl = wm * WTM + i * 16 + lr + r;
        if (MODE == G_ROWS && rl >= mrows) continue;
        const int64_t row = (MODE == G_ROWS) ? int64_t(row0 + rl) : int64_t(m0 + rl);
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int col = n0 + wn * WTN + j * 16 + lc;
          Elem<TC>::store(Cb + row * g.ldc + col, acc[i][j][r]);
        }
      }
  } else if (EPI == EPI_SWIGLU) {
    T* GU = reinterpret_cast<T*>(g.aux0);
    T* H = reinterpret_cast<T*>(g.aux1);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int rl = wm * WTM + i * 16 + lr + r;
        if (rl >= mrows) continue;
        const int64_t row = row0 + rl;
#pragma unroll
        for (int j = 0; j < FN / 2; ++j) {
          const int col = nt * (BN / 2) + wn * (WTN / 2) + j * 16 + lc;
          const float G = acc[i][j][r], U = acc[i][j + FN / 2][r];
          const float Hv = G / (1.0f + expf(-G)) * U;
          Elem<T>::store(GU + row * (2 * g.f) + col, G);
          Elem<T>::store(GU + row * (2 * g.f) + g.f + col, U);
          Elem<T>::store(H + row * g.f + col, Hv);
        }
      }
  } else {  // EPI_DSWIGLU: C = dGU [rows, 2f]
    const T* GU = reinterpret_cast<const T*>(g.aux0);
    T* D = reinterpret_cast<T*>(g.C);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int rl = wm * WTM + i * 16 + lr + r;
        if (rl >= mrows) continue;
        const int64_t row = row0 + rl;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int col = n0 + wn * WTN + j * 16 + lc;
          const float dH = acc[i][j][r];
          const float G = Elem<T>::load(GU + row * (2 * g.f) + col);
          const float U = Elem<T>::load(GU + row * (2 * g.f) + g.f + col);
          const float sg = 1.0f / (1.0f + expf(-G));
          Elem<T>::store(D + row * (2 * g.f) + col, dH * U * sg * (1.0f + G * (1.0f - sg)));
          Elem<T>::store(D + row * (2 * g.f) + g.f + col, dH * G * sg);
        }
      }
  }
}

#undef MOE_GLOAD
#undef MOE_LSTORE

// ---------------------------------------------------------------------------
template <typename T> struct Tile;
template <> struct Tile<bf16_t> { static constexpr int BM = 128, BN = 128, BK = 64; };
template <> struct Tile<float> { static constexpr int BM = 128, BN = 128, BK = 32; };

static int rows_tile_bound(int64_t A, int64_t G, int BM) {
  return int((A + G * (BM - 1)) / BM);
}

template <typename T, typename TC, bool AK, bool BKm, int MODE, int EPI>
static void run_gemm(GemmArgs g, int grid, hipStream_t st) {
  constexpr int BM = Tile<T>::BM, BN = Tile<T>::BN, BK = Tile<T>::BK;
  if (grid <= 0) return;
  gemm_kernel<T, TC, AK, BKm, MODE, EPI, BM, BN, BK, 2, 2><<<grid, 256, 0, st>>>(g);
}

template <typename T>
__global__ void copy_kernel(const T* __restrict__ src, T* __restrict__ dst, int64_t n) {
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < n; i += int64_t(gridDim.x) * blockDim.x)
    dst[i] = src[i];
}

__global__ void zero_kernel(uint32_t* __restrict__ dst, int64_t n) {
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < n; i += int64_t(gridDim.x) * blockDim.x)
    dst[i] = 0u;
}

static void copy_bytes(const void* src, void* dst, int64_t bytes, hipStream_t st) {
  const int64_t n = bytes / 4;
  if (n > 0) copy_kernel<uint32_t><<<1024, 256, 0, st>>>(reinterpret_cast<const uint32_t*>(src),
                                                         reinterpret_cast<uint32_t*>(dst), n);
}

static void zero_bytes(void* dst, int64_t bytes, hipStream_t st) {
  const int64_t n = bytes / 4;
  if (n > 0) zero_kernel<<<1024, 256, 0, st>>>(reinterpret_cast<uint32_t*>(dst), n);
}

template <typename T>
static void ffn_fwd_t(const FfnLaunch& a, hipStream_t st) {
  constexpr int BM = Tile<T>::BM, BN = Tile<T>::BN;
  const int mt_bound = rows_tile_bound(a.A, a.E, BM);
  // GEMM1 + SwiGLU
  GemmArgs g1{};
  g1.A = a.x_perm; g1.lda = a.d;
  g1.B = a.w1; g1.ldb = a.d; g1.b_gstride = 2 * a.f * a.d;
  g1.offsets = a.offsets; g1.G = int(a.E);
  g1.N = int(2 * a.f); g1.K = int(a.d); g1.f = int(a.f);
  g1.aux0 = a.act_gu; g1.aux1 = a.act_h;
  g1.tiles_n = int(2 * a.f / BN);
  run_gemm<T, T, true, true, G_ROWS, EPI_SWIGLU>(g1, mt_bound * g1.tiles_n, st);
  // GEMM2
  GemmArgs g2{};
  g2.A = a.act_h; g2.lda = a.f;
  g2.B = a.w2; g2.ldb = a.f; g2.b_gstride = a.d * a.f;
  g2.C = a.out_perm; g2.ldc = a.d;
  g2.offsets = a.offsets; g2.G = int(a.E);
  g2.N = int(a.d); g2.K = int(a.f);
  g2.tiles_n = int(a.d / BN);
  run_gemm<T, T, true, true, G_ROWS, EPI_STORE>(g2, mt_bound * g2.tiles_n, st);
}

template <typename T>
static void ffn_bwd_t(const FfnBwdLaunch& a, hipStream_t st) {
  constexpr int BM = Tile<T>::BM, BN = Tile<T>::BN;
  const int mt_bound = rows_tile_bound(a.A, a.E, BM);
  // dH = dO W2, fused SwiGLU backward -> dGU
  GemmArgs g1{};
  g1.A = a.d_out; g1.lda = a.d;
  g1.B = a.w2; g1.ldb = a.f; g1.b_gstride = a.d * a.f;
  g1.C = a.d_gu; g1.ldc = 2 * a.f;
  g1.offsets = a.offsets; g1.G = int(a.E);
  g1.N = int(a.f); g1.K = int(a.d); g1.f = int(a.f);
  g1.aux0 = const_cast<void*>(a.act_gu);
  g1.tiles_n = int(a.f / BN);
  run_gemm<T, T, true, false, G_ROWS, EPI_DSWIGLU>(g1, mt_bound * g1.tiles_n, st);
  // dX = dGU W1
  GemmArgs g2{};
  g2.A = a.d_gu; g2.lda = 2 * a.f;
  g2.B = a.w1; g2.ldb = a.d; g2.b_gstride = 2 * a.f * a.d;
  g2.C = a.dx_perm; g2.ldc = a.d;
  g2.offsets = a.offsets; g2.G = int(a.E);
  g2.N = int(a.d); g2.K = int(2 * a.f);
  g2.tiles_n = int(a.d / BN);
  run_gemm<T, T, true, false, G_ROWS, EPI_STORE>(g2, mt_bound * g2.tiles_n, st);
  // dW2 = dO^T H   [d, f]
  GemmArgs g3{};
  g3.A = a.d_out; g3.lda = a.d;
  g3.B = a.act_h; g3.ldb = a.f;
  g3.C = a.dw2; g3.ldc = a.f; g3.c_gstride = a.d * a.f;
  g3.offsets = a.offsets; g3.G = int(a.E);
  g3.M = int(a.d); g3.N = int(a.f);
  g3.tiles_m = int(a.d / BM); g3.tiles_n = int(a.f / BN);
  run_gemm<T, T, false, false, G_KSPLIT, EPI_STORE>(g3, int(a.E) * g3.tiles_m * g3.tiles_n, st);
  // dW1 = dGU^T X   [2f, d]
  GemmArgs g4{};
  g4.A = a.d_gu; g4.lda = 2 * a.f;
  g4.B = a.x_perm; g4.ldb = a.d;
  g4.C = a.dw1; g4.ldc = a.d; g4.c_gstride = 2 * a.f * a.d;
  g4.offsets = a.offsets; g4.G = int(a.E);
  g4.M = int(2 * a.f); g4.N = int(a.d);
  g4.tiles_m = int(2 * a.f / BM); g4.tiles_n = int(a.d / BN);
  run_gemm<T, T, false, false, G_KSPLIT, EPI_STORE>(g4, int(a.E) * g4.tiles_m * g4.tiles_n, st);
}

void launch_grouped_ffn(const FfnLaunch& a, hipStream_t st) {
  if (a.identity) {
    copy_bytes(a.x_perm, a.out_perm, a.A * a.d * (a.act == 1 ? 2 : 4), st);
    return;
  }
  if (a.wt == 1) ffn_fwd_t<bf16_t>(a, st);
  else ffn_fwd_t<float>(a, st);
}

void launch_grouped_ffn_bwd(const FfnBwdLaunch& a, hipStream_t st) {
  const int es = (a.act == 1 ? 2 : 4);
  if (a.identity) {
    copy_bytes(a.d_out, a.dx_perm, a.A * a.d * es, st);
    const int ws = (a.wt == 0 ? 4 : 2);
    zero_bytes(a.dw1, a.E * 2 * a.f * a.d * ws, st);
    zero_bytes(a.dw2, a.E * a.d * a.f * ws, st);
    return;
  }
  if (a.wt == 1) ffn_bwd_t<bf16_t>(a, st);
  else ffn_bwd_t<float>(a, st);
}

}  // namespace moe

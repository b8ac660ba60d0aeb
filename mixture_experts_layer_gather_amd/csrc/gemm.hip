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
// in fp32 (v_mfma_f32_16x16x4f32), bf16 (v_mfma_f32_16x16x32_bf16) and FP8
// E4M3 (v_mfma_scale_f32_16x16x128_f8f6f4 with unit hardware scales). FP8
// operands carry fp32 block scales (activations 1 x 128 along K, weights
// 128 x 128): a K step is exactly one 128-deep block, its MFMA result is
// multiplied by row scale x column-block scale and added to the fp32
// accumulator. MXFP8 operands (mx8_t) carry one E8M0 byte per 32 K-values,
// which the same instruction applies itself (hardware scales per lane).
// The SwiGLU epilogues can skip saving GU and rebuild H in the backward
// (activation recompute).
//
// Tiles go global -> LDS by DMA (2 or 3 stages, one barrier per K step).
// K-major operands land in K-contiguous rows and are read with 16-byte LDS
// reads; K-strided bf16 and FP8 operands land in their source orientation
// and are read with the LDS transpose reads; only K-strided fp32 operands are
// transposed in registers on their way into LDS. Workgroup ids are remapped
// so that each XCD (8 per chip, one L2 each) works through a contiguous range
// of tiles that share weights and rows.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace moe {

enum { G_ROWS = 0, G_KSPLIT = 1 };

// Compile-time loop: f(std::integral_constant<int, I>) for I = 0 .. N-1.
template <int I, int N> struct StaticFor {
  template <typename F> __device__ __forceinline__ static void run(F& f) {
    f(std::integral_constant<int, I>{});
    StaticFor<I + 1, N>::run(f);
  }
};
template <int N> struct StaticFor<N, N> {
  template <typename F> __device__ __forceinline__ static void run(F&) {}
};
template <int N, typename F> __device__ __forceinline__ void static_for(F&& f) { StaticFor<0, N>::run(f); }
enum { EPI_STORE = 0, EPI_SWIGLU = 1, EPI_DSWIGLU = 2 };

typedef uint8_t fp8_t;  // OCP E4M3FN code
// MXFP8 operand: E4M3 codes whose scales are E8M0 bytes per 32 K-values,
// applied by the matrix core itself (a distinct type selects that path)
enum class mx8_t : uint8_t {};

template <typename T> struct Mfma;
template <> struct Mfma<bf16_t> {
  static constexpr int KP = 8;   // elements per lane per instruction
  static constexpr int MK = 32;  // K per instruction
  typedef bf16x8_t frag;
  // K offset (within the LDS tile) of lane's fragment for sub-step kk
  static __device__ __forceinline__ int kofs(int lane, int kk) { return kk * MK + (lane / 16) * KP; }
  static constexpr int K2 = 0;   // offset of the second 16-byte chunk (unused)
  static __device__ __forceinline__ frag load(const bf16_t* p0, const bf16_t*) {
    return __builtin_bit_cast(frag, *reinterpret_cast<const u32x4*>(p0));
  }
  static __device__ __forceinline__ f32x4_t mma(frag a, frag b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mfma<float> {
  static constexpr int KP = 1;
  static constexpr int MK = 4;
  typedef float frag;
  static __device__ __forceinline__ int kofs(int lane, int kk) { return kk * MK + lane / 16; }
  static constexpr int K2 = 0;
  static __device__ __forceinline__ frag load(const float* p0, const float*) { return *p0; }
  static __device__ __forceinline__ f32x4_t mma(frag a, frag b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};
template <> struct Mfma<fp8_t> {
  static constexpr int KP = 32;
  static constexpr int MK = 128;
  typedef i32x8_t frag;
  // The 32 K-values a lane feeds are chunks q and q + 4 (q = lane / 16) of the
  // 128-deep block, not 2q and 2q + 1: A and B use the same order, so every
  // product is still formed, and the LDS reads then follow the conflict-free
  // pattern of the bf16 fragments (16 rows x 4 consecutive chunks).
  static __device__ __forceinline__ int kofs(int lane, int) { return (lane / 16) * 16; }
  static constexpr int K2 = 64;
  // 32 bytes from two (separately swizzled) 16-byte chunks
  static __device__ __forceinline__ frag load(const fp8_t* p0, const fp8_t* p1) {
    const u32x4 lo = *reinterpret_cast<const u32x4*>(p0);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(p1);
    return i32x8_t{int(lo[0]), int(lo[1]), int(lo[2]), int(lo[3]),
                   int(hi[0]), int(hi[1]), int(hi[2]), int(hi[3])};
  }
  // A and B formats 0 (E4M3), E8M0 hardware scales 127 (= 1.0)
  static __device__ __forceinline__ f32x4_t mma(frag a, frag b, f32x4_t c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
  }
};

// MXFP8: the same fragments. In the matrix core's K order a lane of group
// q = l / 16 feeds K-values 16q .. 16q + 15 and 64 + 16q .. 64 + 16q + 15 of
// the 128-deep block, and the scale byte of lane l (row or column l % 16)
// applies to K block q, i.e. K-values 32q .. 32q + 31, held by groups 2q % 4
// and (2q + 1) % 4 (measured on gfx950 with one wave and marked scales). The
// operands' K order in LDS is the source order, so block q of a row is MXFP8
// block 4 s + q of step s.
template <> struct Mfma<mx8_t> : Mfma<fp8_t> {
  static __device__ __forceinline__ frag load(const mx8_t* p0, const mx8_t* p1) {
    return Mfma<fp8_t>::load(reinterpret_cast<const fp8_t*>(p0), reinterpret_cast<const fp8_t*>(p1));
  }
  static __device__ __forceinline__ f32x4_t mma_scaled(frag a, frag b, f32x4_t c, int sa, int sb) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
  }
};

// Activation dtype of the epilogue outputs for operand dtype T.
template <typename T> struct OutOf { typedef T type; };
template <> struct OutOf<fp8_t> { typedef bf16_t type; };
template <> struct OutOf<mx8_t> { typedef bf16_t type; };


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
  void* aux0;         // SWIGLU: GU out [rows,2f] or null (not kept); DSWIGLU: GU in
  void* aux1;         // SWIGLU: H out [rows,f]; DSWIGLU: H recomputed out, or null
  int tiles_n;
  int tiles_m;        // KSPLIT
  // FP8 block scales
  const float* a_scale;      // [rows, K/128]
  int a_scale_ld;            // K/128
  const float* b_scale;      // [G, R/128, C/128] of B's storage [G, R, C]
  int64_t b_scale_gstride;   // (R/128)*(C/128)
  int b_scale_ld;            // C/128
  // FP8 weight gradients: operands quantised in 128-row x 1 blocks inside
  // each group's rows; a_scale [NB, M] and b_scale [NB, N] (row lengths
  // a_scale_ld = M, b_scale_ld = N) hold one scale per block and column, and
  // kblk[g] is the first block of group g (kblk[G] = NB)
  const int32_t* kblk;
  int tpw;                   // FP8 weight gradients: column tiles per workgroup
  int ksuper;                // tiles per XCD super-block (set by run_gemm)
};

// Workgroup id -> tile. Consecutive ids are dispatched to the 8 XCDs round
// robin (one L2 each). Tiles are dealt to XCDs in super-blocks of ks
// consecutive tiles: XCD x takes super-blocks x, x+8, x+16, ... so tiles
// that share operands (same expert, neighbouring row/column blocks) run on
// one L2, while a hot expert's many super-blocks spread over all XCDs. The
// grid is a multiple of 8*ks, which makes the map a bijection.
__device__ __forceinline__ int tile_remap(int bid, int ks) {
  const int x = bid % 8, i = bid / 8;
  return ((i / ks) * 8 + x) * ks + (i % ks);
}
static int padded_grid(int tiles, int ks) {
  const int q = 8 * ks;
  return (tiles + q - 1) / q * q;
}
// Super-block sizes, measured (per-launch times on the Mixtral-, Qwen3- and
// DeepSeek-style layers against 64 everywhere):
//   row-grouped GEMMs on the 128 x 128 tile: 32 (Mixtral dX 2.41 -> 2.29 ms,
//     DeepSeek GEMM1 3.89 -> 3.81 ms, the others within noise);
//   on the 256 x 256 tile: 64, and 32 when experts average at least 128
//     tiles (Mixtral-style GEMM1 and dH: step 9.41 -> 9.34 ms; the
//     Qwen3-style GEMM1, about 30 tiles per expert, loses 3 % with 32);
//   weight gradients: 16 when an expert has fewer than 256 tiles (so that a
//     super-block stays inside one expert; Qwen3-style 0.91 -> 0.78 ms), else
//     64 (16 costs the DeepSeek-style layer 4 %).
//   and 16 for row-grouped GEMMs whose experts average fewer than 16 tiles
//     (Qwen3-style dH, 3 column tiles per expert: 0.73 -> 0.65 ms).
constexpr int kSuperRowsSmall = 32, kSuperRowsBig = 64;
static int super_wgrad(int tiles_per_group) { return tiles_per_group < 256 ? 16 : 64; }
static int super_rows(int tiles_per_group, int bm) {
  if (tiles_per_group < 16) return 16;
  if (bm < 256) return kSuperRowsSmall;
  return tiles_per_group >= 128 ? 32 : kSuperRowsBig;
}

// Exclusive scan of per-group row-tile counts; returns the tile's group in
// s_info[0], its row-tile count in s_info[1] and the first tile of the group
// in s_info[2], or s_info[0] = -1 when the tile is past the end.
template <int BM, int NTH>
__device__ void find_group(const int32_t* __restrict__ offsets, int G, int tiles_n, int tile,
                           int* s_scan, int* s_info) {
  const int tid = threadIdx.x;
  constexpr int PER = 1024 / NTH;  // groups per thread (G <= 1024)
  int cnt[PER], local = 0;
  // the PER + 1 offsets go out together (a group past G reads offsets[G],
  // in bounds, and counts nothing); under a per-group branch each load was
  // waited for alone
  int off[PER + 1];
#pragma unroll
  for (int i = 0; i <= PER; ++i) off[i] = offsets[min(tid * PER + i, G)];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int g = tid * PER + i;
    const int c = g < G ? (off[i + 1] - off[i] + BM - 1) / BM : 0;
    cnt[i] = c;
    local += c;
  }
  // inclusive scan of `local` across the NTH threads
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

// LDS tiles hold ROWS x BK elements per operand (rows of 128 or 64 bytes),
// K-contiguous, without padding; the 16-byte chunks of a row are XOR-swizzled
// with the row. Measured with the LDS bank-conflict counters on gfx950: the
// MFMA fragment reads (16 consecutive rows x 4 chunks per instruction) of
// 128-byte rows are conflict-free when the swizzle takes row bits 0-2 (and
// not row bit 3); for 64-byte rows, row bits 1-2; 16-byte row stores are
// conflict-free for any swizzle; the transposed 8-byte stores of K-strided
// operands (128-byte rows only) need rows 8 and 16 apart to differ, which
// row bits 4-6 provide. So K-major operands (filled by DMA) use the low row
// bits only, which keeps a fragment's address an immediate offset from the
// first fragment's, and K-strided operands add row bits 4-6.
template <bool KMAJ, int NCH>
__device__ __forceinline__ int lds_swz(int row) {
  static_assert(NCH == 8 || (NCH == 4 && KMAJ), "128-byte rows, or 64-byte K-major rows");
  if constexpr (NCH == 4) return (row >> 1) & 3;
  return KMAJ ? (row & 7) : ((row ^ (row >> 4)) & 7);
}
template <typename T, int BK, bool KMAJ>
__device__ __forceinline__ int lds_off(int row, int k) {
  constexpr int VEC = 16 / sizeof(T);
  constexpr int NCH = BK / VEC;
  return row * BK + (((k / VEC) ^ lds_swz<KMAJ, NCH>(row)) * VEC) + (k % VEC);
}

// fp32: 4 K-rows x 4 columns (four 16-byte registers) -> 4 LDS rows of 4
// K-values each (the only register-transposed operands: K-strided bf16 and
// FP8 tiles are read with the LDS transpose reads instead).
template <typename T, int BK>
__device__ __forceinline__ void store_transposed(const u32x4* r, T* dst, int c0, int k4) {
  static_assert(sizeof(T) == 4, "register transposes serve fp32 operands only");
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const u32x4 v = {r[0][c], r[1][c], r[2][c], r[3][c]};
    *reinterpret_cast<u32x4*>(dst + lds_off<T, BK, false>(c0 + c, k4)) = v;
  }
}

// Raw buffer descriptors (gfx9 family: stride 0, 32-bit untyped data). A
// load whose byte offset lies at or past `bytes` returns zeros, which masks
// rows past the end of a group without branches. The range field is 32 bits:
// a longer remaining range is clamped to 2^32 - 1, which masks nothing that
// a load of the step can reach (every offset a step uses is a 32-bit offset
// from the step's own base, and the host rejects shapes whose per-step
// offsets could pass 4 GiB).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ uint32_t rsrc_range(int64_t bytes) {
  return bytes <= 0 ? 0u : (bytes >= int64_t(0xffffffff) ? 0xffffffffu : uint32_t(bytes));
}
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(rsrc_range(bytes)), 0x00020000);
}
// One wave instruction of DMA: every lane's 16 bytes at byte offset voff of
// the buffer described by rsrc go to LDS at dst + 16 * lane (dst is
// wave-uniform). Issued as inline assembly on purpose: the compiler then does
// not track it as an LDS write and inserts no wait for it before LDS reads
// (it cannot tell the transpose-read intrinsic apart from the stage being
// filled, and would wait for the prefetch of the next K step there). The K
// loop therefore waits for its DMA explicitly (vmcnt) before each barrier.
__device__ __forceinline__ u32x4 rsrc_words(const void* base, int64_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return u32x4{uint32_t(a), uint32_t(a >> 32) & 0xffffu, rsrc_range(bytes), 0x00020000u};
}
__device__ __forceinline__ void dma16(u32x4 rsrc, void* dst, uint32_t voff) {
  const uint32_t lds = uint32_t(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)dst));
  asm volatile("s_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %0, %2, 0 offen lds"
               :
               : "v"(voff), "s"(lds), "s"(rsrc)
               : "memory", "m0");
}
// The same with 4 bytes per lane (lane l's dword to LDS at dst + 4 * l): a
// gather of one value per row, such as FP8 row scales.
__device__ __forceinline__ void dma4(u32x4 rsrc, void* dst, uint32_t voff) {
  const uint32_t lds = uint32_t(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)dst));
  asm volatile("s_mov_b32 m0, %1\n\tbuffer_load_dword %0, %2, 0 offen lds"
               :
               : "v"(voff), "s"(lds), "s"(rsrc)
               : "memory", "m0");
}
// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maxima)
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0f70); }
// the s_waitcnt immediate for vmcnt(n), n < 64
constexpr int vm_wait(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Operand tiles in LDS, by layout mode:
//   LM_KDMA  K-major source, DMA straight from global memory into ROWS rows of
//            BK elements (128 bytes). One wave instruction fills 1 KB of LDS
//            = 8 rows, lane l the 16 bytes at l * 16; the lane fetches the
//            logical chunk that the swizzle puts there.
//   LM_TDMA  K-strided bf16 source, DMA into BK K-rows of ROWS elements (the
//            source's own orientation); 16-byte chunks are XOR-swizzled with
//            tr_swz(K-row). MFMA fragments are read with the LDS transpose
//            read (ds_read_b64_tr_b16), which hands each lane of a 16-lane
//            group one column of 4 consecutive K-rows. Measured on gfx950,
//            the transpose read serves 32 lanes (two groups, K-rows 8 apart)
//            at a time: the swizzle separates the 4 K-rows of a group (bits
//            1-2) and the two groups (bit 3), which makes it conflict-free.
//            FP8 (128-byte K-rows, 8 chunks): chunks are XOR-swizzled with
//            tr8_swz(K-row) and fragments are read with ds_read_b64_tr_b8,
//            which gives lane i of a 16-lane group, byte j, element i % 8 of
//            the 8 bytes addressed by lane 2 j + i / 8 (measured on gfx950):
//            lanes 2 j and 2 j + 1 address the two 8-column halves of K-row
//            j, so a lane receives its column of 8 consecutive K-rows. The
//            swizzle gives the 16 K-rows that two groups read together 16
//            distinct bank windows.
//   LM_REG   other K-strided sources (fp32): NT blocks of 4 K-rows x VEC
//            columns per thread, loaded into registers and transposed on
//            their way into LDS (K-major rows, swizzled as in lds_off).
enum { LM_KDMA = 0, LM_TDMA = 1, LM_REG = 2 };
template <typename T, bool KMAJ>
constexpr int layout_mode() {
  return KMAJ ? LM_KDMA : (sizeof(T) <= 2 ? LM_TDMA : LM_REG);
}

template <typename T, int LM, int ROWS, int BK, int NTH>
struct OperandPlan {
  static constexpr int VEC = 16 / sizeof(T);
  static constexpr int NW = NTH / 64;
  static constexpr int NB = ROWS * BK * int(sizeof(T)) / 1024 / NW;  // DMA instructions per wave
  static constexpr int NT = BK * ROWS / (4 * VEC) / NTH;               // LM_REG blocks per thread
  static constexpr bool DMA = LM != LM_REG;
  static constexpr int NREG = DMA ? 1 : 4 * NT;
  static_assert(!DMA || NB * 1024 * NW == ROWS * BK * int(sizeof(T)), "DMA blocks per wave");
  static_assert(DMA || (NT >= 1 && NT * 4 * VEC * NTH == ROWS * BK), "tile/threads");
  static_assert(LM != LM_TDMA || (sizeof(T) == 2 && ROWS * 2 >= 256 && 1024 % (ROWS * 2) == 0) ||
                    (sizeof(T) == 1 && (ROWS == 128 || ROWS == 256)),
                "transposed tiles: bf16 rows of 256 or 512 bytes (at least 16 chunks for the swizzle), "
                "FP8 rows of 128 bytes");
  uint32_t voff[DMA ? NB : 4 * NT];  // byte offsets from the step's base
  int lrow[DMA ? 1 : NT];            // LM_REG: first LDS row of the block
  int lk[DMA ? 1 : NT];              // LM_REG: LDS k offset
};

__device__ __forceinline__ int tr_swz(int kr) { return (2 * (kr & 3)) ^ (8 * ((kr >> 3) & 1)); }
// FP8 K-rows of 8 chunks: K-rows 0, 2, 4, 6, 16, 18, 20, 22 (and the odd ones,
// which sit in the other half of the banks) get chunk masks 0 .. 7
__device__ __forceinline__ int tr8_swz(int kr) { return ((kr >> 1) & 3) | ((kr >> 2) & 4); }
// FP8 K-rows of 16 chunks (256-byte rows: each K-row covers every bank): the
// 16 K-rows two 16-lane groups read together (K-rows j and 16 + j, j < 8,
// plus a common offset of 8 or 64) get 16 distinct chunk masks
__device__ __forceinline__ int tr8w_swz(int kr) { return (kr & 7) | ((kr >> 1) & 8); }
template <int ROWS>
__device__ __forceinline__ int tr8_swz_rows(int kr) {
  if constexpr (ROWS == 256) return tr8w_swz(kr);
  return tr8_swz(kr);
}

// 8 consecutive values: fp32 from LDS; bf16 / fp32 to and from global memory
__device__ __forceinline__ void lds_read8(const float* p, float* v) {
  const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
template <typename T> __device__ __forceinline__ void store8(T* p, const float* v) {
  if constexpr (sizeof(T) == 2) {
    Vec16<bf16_t>::store(p, v);
  } else {
    Vec16<float>::store(p, v);
    Vec16<float>::store(p + 4, v + 4);
  }
}
template <typename T> __device__ __forceinline__ void store8_stream(T* p, const float* v) {
  if constexpr (sizeof(T) == 2) {
    st_stream(p, Vec16<bf16_t>::pack(v));
  } else {
    st_stream(p, Vec16<float>::pack(v));
    st_stream(p + 4, Vec16<float>::pack(v + 4));
  }
}
// Rounds 8 values to the storage type T and back (the values as saved).
template <typename T> __device__ __forceinline__ void round8(float* v) {
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = bf16_to_f32(f32_to_bf16(v[e]));
  }
}
// SwiGLU output from the gate and up values as saved; the forward and the
// backward's recompute share this expression, so both give the same bits.
__device__ __forceinline__ float swiglu_h(float g, float u) { return g / (1.0f + expf(-g)) * u; }
template <typename T> __device__ __forceinline__ void load8(const T* p, float* v) {
  if constexpr (sizeof(T) == 2) {
    Vec16<bf16_t>::load(p, v);
  } else {
    Vec16<float>::load(p, v);
    Vec16<float>::load(p + 4, v + 4);
  }
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
// LDS transpose read of 16-bit data: in each 16-lane group, slot j of lane i
// receives element i % 4 of the 8 bytes addressed by lane 4 j + i / 4.
__device__ __forceinline__ u32x2 lds_read_tr16(const void* p) {
  return __builtin_bit_cast(
      u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(void*)p));
}

// One LDS stage (operand tiles and FP8 row scales).
template <typename T, int BM, int BN, int BK, int NTH, bool SCALED>
struct alignas(16) Stage {  // 16-byte multiple: stages sit back to back in one array
  T A[BM * BK];
  T B[BN * BK];
  float SA[SCALED ? (NTH > BM ? NTH : BM) : 1];  // FP8 row scales of the A tile (padded)
};
// MXFP8 stage: per A row and per B column, the E8M0 bytes of the step's four
// 32-deep K blocks in one word (byte q = block q)
template <int BM, int BN, int BK, int NTH>
struct alignas(16) StageMx {
  mx8_t A[BM * BK];
  mx8_t B[BN * BK];
  uint32_t SA[NTH > BM ? NTH : BM];
  uint32_t SB[NTH > BN ? NTH : BN];
};

// The weight-gradient instances that run persistent runs of column tiles:
// FP8 or MXFP8 operands (token-block scales), or bf16 operands on the
// two-stage 128 x 128 tile; bf16 results. (The host takes the bf16 one only
// for experts of a few hundred rows: with long K the 128 x 256 three-stage
// tile wins, Qwen3-style dW1 0.95 vs 2.17 ms, Mixtral-style 2.15 vs 2.55 ms.)
template <typename T, typename TC, int MODE, int EPI, int NS>
constexpr bool persistent_wgrad() {
  return MODE == G_KSPLIT && EPI == EPI_STORE && NS == 2 && sizeof(TC) == 2 &&
         (std::is_same<T, fp8_t>::value || std::is_same<T, mx8_t>::value || std::is_same<T, bf16_t>::value);
}

template <typename T, typename TC, bool A_KMAJ, bool B_KMAJ, int MODE, int EPI, int BM, int BN,
          int BK, int WM, int WN, int NS>
__global__ __launch_bounds__(WM * WN * 64) __attribute__((amdgpu_waves_per_eu(2)))
void gemm_kernel(GemmArgs g) {
  constexpr int NTH = WM * WN * 64;
  using MF = Mfma<T>;
  using TO = typename OutOf<T>::type;
  constexpr bool FP8 = sizeof(T) == 1;
  constexpr bool MX = std::is_same<T, mx8_t>::value;
  // 8-bit weight gradients: a scale per (128-row block, column) of both
  // operands, staged per K step with the tiles (TOKW): FP8 fp32 scales,
  // applied by VALU FMAs (TOKSCALE), or MXFP8 words of the block's four
  // 32-row E8M0 bytes, applied by the matrix core (TOKMX)
  constexpr bool TOKSCALE = FP8 && !MX && MODE == G_KSPLIT;
  constexpr bool TOKMX = MX && MODE == G_KSPLIT;
  constexpr bool TOKW = TOKSCALE || TOKMX;
  using ST = std::conditional_t<MX, StageMx<BM, BN, BK, WM * WN * 64>, Stage<T, BM, BN, BK, WM * WN * 64, FP8>>;
  constexpr int VEC = 16 / sizeof(T);
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 16, FN = WTN / 16;
  constexpr int ALM = layout_mode<T, A_KMAJ>(), BLM = layout_mode<T, B_KMAJ>();
  using PA = OperandPlan<T, ALM, BM, BK, NTH>;
  using PB = OperandPlan<T, BLM, BN, BK, NTH>;
  // weight gradients as runs of column tiles per workgroup (8-bit operands)
  constexpr bool PERSIST = persistent_wgrad<T, TC, MODE, EPI, NS>();
  static_assert(!PERSIST || (PA::DMA && PB::DMA), "persistent weight gradients load by DMA");
  static_assert(WM * WN == 4 || WM * WN == 8, "four or eight waves");
  static_assert(EPI != EPI_SWIGLU || FN % 2 == 0, "SwiGLU pairs column fragments");
  static_assert(!FP8 || (MODE == G_ROWS && A_KMAJ && BK == 128 && BN <= 256 && BM <= 256) ||
                    (TOKW && PERSIST && !A_KMAJ && !B_KMAJ && BK == 128 && BM + BN <= WM * WN * 64),
                "FP8: row-grouped GEMMs, or weight gradients, one 128-deep scale block per K step");

  static_assert(NS >= 2 && NS <= 4, "LDS stages");
  static_assert(sizeof(ST) % 16 == 0, "stage alignment");
  __shared__ __attribute__((aligned(16))) ST stv[NS];
  ST& st0 = stv[0];
  ST& st1 = stv[1];
  __shared__ int s_scan[8];
  __shared__ int s_info[3];

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave / WN, wn = wave % WN;
  const int tile = tile_remap(blockIdx.x, g.ksuper);

  // tile -> (group, row tile, column tile); all of it wave-uniform
  int grp, mt, nt;
  int row0;           // first A row (ROWS) of the tile
  int mrows;          // valid rows in the tile (ROWS)
  int kbase, kcount;  // contraction range
  if (MODE == G_ROWS) {
    find_group<BM, NTH>(g.offsets, g.G, g.tiles_n, tile, s_scan, s_info);
    grp = __builtin_amdgcn_readfirstlane(s_info[0]);
    if (grp < 0) return;
    const int cnt = __builtin_amdgcn_readfirstlane(s_info[1]);
    const int local = tile - __builtin_amdgcn_readfirstlane(s_info[2]);
    nt = local / cnt;
    mt = local % cnt;
    row0 = g.offsets[grp] + mt * BM;
    mrows = min(BM, g.offsets[grp + 1] - row0);
    kbase = 0;
    kcount = g.K;
  } else if constexpr (PERSIST) {
    // a run of up to tpw consecutive column tiles of one (group, row block);
    // runs fastest, so that the workgroups running at once write
    // neighbouring runs of the same rows: the write front covers whole rows
    // instead of 256-byte pieces of many rows (row blocks fastest measured
    // 6 % slower on dW1, FP8 and bf16)
    const int tpw = max(g.tpw, 1);
    const int nch = (g.tiles_n + tpw - 1) / tpw;
    const int per = g.tiles_m * nch;
    grp = tile / per;
    if (grp >= g.G) return;  // padding of the grid
    const int rem = tile % per;
    nt = (rem % nch) * tpw;
    mt = rem / nch;
    row0 = 0;
    mrows = BM;
    kbase = g.offsets[grp];
    kcount = g.offsets[grp + 1] - kbase;
  } else {
    const int per = g.tiles_m * g.tiles_n;
    grp = tile / per;
    if (grp >= g.G) return;  // padding of the grid
    // bands of 8 row tiles, row tile fastest: a super-block of ks
    // consecutive tiles covers 8 x (ks / 8) tiles, sharing each A panel
    // ks / 8 times and each B panel 8 times
    const int rem = tile % per;
    const int band = rem / (8 * g.tiles_n);
    const int in_band = min(8, g.tiles_m - band * 8);
    const int idx = rem - band * 8 * g.tiles_n;
    mt = band * 8 + idx % in_band;
    nt = idx / in_band;
    row0 = 0;
    mrows = BM;
    kbase = g.offsets[grp];
    kcount = g.offsets[grp + 1] - kbase;
  }
  const int m0 = mt * BM;  // KSPLIT: output row block
  const int n0 = nt * BN;
  const int nk = (kcount + BK - 1) / BK;  // K steps
  constexpr int64_t ES = sizeof(T);

  // ---- operand sources: byte base at K step 0, byte end of the valid
  // range, byte advance per K step
  const char* a_base;
  int64_t a_end, a_step;
  if constexpr (A_KMAJ) {  // rows row0 .. row0 + mrows of A [rows, K]
    a_base = reinterpret_cast<const char*>(g.A) + int64_t(row0) * g.lda * ES;
    a_end = int64_t(mrows) * g.lda * ES;
    a_step = BK * ES;
  } else {  // K-rows kbase .. kbase + kcount of A [K, M]
    a_base = reinterpret_cast<const char*>(g.A) + int64_t(kbase) * g.lda * ES;
    a_end = int64_t(kcount) * g.lda * ES;
    a_step = BK * g.lda * ES;
  }
  const char* b_base = reinterpret_cast<const char*>(g.B);
  if (MODE == G_ROWS) b_base += int64_t(grp) * g.b_gstride * ES;
  int64_t b_end, b_step;
  if constexpr (B_KMAJ) {  // rows 0 .. N of B [N, K] (ROWS)
    b_end = int64_t(g.N) * g.ldb * ES;
    b_step = BK * ES;
  } else if constexpr (MODE == G_ROWS) {  // B [K, N]
    b_end = int64_t(g.K) * g.ldb * ES;
    b_step = BK * g.ldb * ES;
  } else {  // K-rows kbase .. kbase + kcount of B [K, N]
    b_base += int64_t(kbase) * g.ldb * ES;
    b_end = int64_t(kcount) * g.ldb * ES;
    b_step = BK * g.ldb * ES;
  }

  // ---- per-thread load plans (offsets are fixed for the whole K loop)
  constexpr int RB = BK * int(ES);   // bytes per K-major LDS row
  constexpr int NCH = RB / 16;       // 16-byte chunks per K-major LDS row
  PA pa;
  PB pb;
  // LM_TDMA: K-row kr of the tile holds ROWS elements from column col0; DMA
  // block b covers K-rows b * RPB .. + RPB
  auto tdma_voff = [&](int b, int ROWS, int64_t ld, int col0) {
    constexpr int EPC = 16 / int(ES);  // elements per 16-byte chunk
    const int CPR = ROWS / EPC, RPB = 1024 / (ROWS * int(ES));
    const int kr = b * RPB + lane / CPR;
    const int lc = (lane % CPR) ^ (ES == 1 ? (ROWS == 256 ? tr8w_swz(kr) : tr8_swz(kr)) : tr_swz(kr));
    return uint32_t((int64_t(kr) * ld + col0 + lc * EPC) * ES);
  };
  if constexpr (ALM == LM_KDMA) {
#pragma unroll
    for (int j = 0; j < PA::NB; ++j) {
      const int r = (j * PA::NW + wave) * (1024 / RB) + lane / NCH;
      const int lc = (lane % NCH) ^ lds_swz<true, NCH>(r);
      pa.voff[j] = uint32_t(int64_t(r) * g.lda * ES + lc * 16);
    }
  } else if constexpr (ALM == LM_TDMA) {
#pragma unroll
    for (int j = 0; j < PA::NB; ++j) pa.voff[j] = tdma_voff(j * PA::NW + wave, BM, g.lda, m0);
  } else {
#pragma unroll
    for (int i = 0; i < PA::NT; ++i) {
      const int q = tid + i * NTH;
      const int kq = q / (BM / VEC), mc = q % (BM / VEC);
      pa.lrow[i] = mc * VEC;
      pa.lk[i] = 4 * kq;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        pa.voff[4 * i + j] = uint32_t((int64_t(4 * kq + j) * g.lda + m0 + mc * VEC) * ES);
    }
  }
  if constexpr (BLM == LM_KDMA) {
#pragma unroll
    for (int j = 0; j < PB::NB; ++j) {
      const int r = (j * PB::NW + wave) * (1024 / RB) + lane / NCH;
      const int lc = (lane % NCH) ^ lds_swz<true, NCH>(r);
      int grow = n0 + r;
      if (EPI == EPI_SWIGLU) {
        // gate and up rows of the same output columns side by side within
        // each wave's column range
        const int w = r / WTN, within = r % WTN;
        const int half = within / (WTN / 2), jj = within % (WTN / 2);
        grow = half * g.f + nt * (BN / 2) + w * (WTN / 2) + jj;
      }
      pb.voff[j] = uint32_t(int64_t(grow) * g.ldb * ES + lc * 16);
    }
  } else if constexpr (BLM == LM_TDMA) {
#pragma unroll
    for (int j = 0; j < PB::NB; ++j) pb.voff[j] = tdma_voff(j * PB::NW + wave, BN, g.ldb, n0);
  } else {
#pragma unroll
    for (int i = 0; i < PB::NT; ++i) {
      const int q = tid + i * NTH;
      const int kq = q / (BN / VEC), nc = q % (BN / VEC);
      pb.lrow[i] = nc * VEC;
      pb.lk[i] = 4 * kq;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        pb.voff[4 * i + j] = uint32_t((int64_t(4 * kq + j) * g.ldb + n0 + nc * VEC) * ES);
    }
  }
  // FP8: thread tid stages the row scale of A-tile row tid; rows past the
  // group (and threads past the tile) read zeros. MXFP8: the same word holds
  // the row's four E8M0 bytes of the step (a_scale_ld = K / 128 words).
  const char* sa_base = nullptr;
  int64_t sa_end = 0;
  if constexpr (FP8 && !TOKW) {
    sa_base = reinterpret_cast<const char*>(g.a_scale + int64_t(row0) * g.a_scale_ld);
    sa_end = int64_t(mrows) * g.a_scale_ld * 4;
  }
  // weight gradients: K step s is block kb0 + s of the scale arrays; its
  // scales land in LDS by DMA, 64 consecutive ones per wave: the A scales of
  // output rows m0 .. m0 + BM (waves below BM / 64), then the B scales of
  // columns n0 .. n0 + BN
  static_assert(!TOKW || (BM % 64 == 0 && BN % 64 == 0 && BM + BN == NTH), "one scale run per wave");
  int kb0 = 0;
  const float* ts_run = nullptr;
  int64_t ts_ld = 0;
  if constexpr (TOKW) {
    kb0 = g.kblk[grp];
    if (wave * 64 < BM) {
      ts_run = g.a_scale + m0 + wave * 64;
      ts_ld = g.a_scale_ld;
    } else {
      ts_run = g.b_scale + n0 + (wave * 64 - BM);
      ts_ld = g.b_scale_ld;
    }
  }
  // FP8: column-block scale rows of B; SwiGLU tiles span a gate block and an
  // up block of W1
  // They travel one step ahead with the row scales, into SA[BM + q] (q < NQB):
  // lane q of each wave past the A rows fetches block q's scale of the step
  // (SwiGLU: q = 0 gate, 1 up; otherwise column block n0 / 128 + q). Read at
  // the step itself, a global load would make the wait for it also wait for
  // the next step's prefetch (loads complete in issue order).
  constexpr int NQB = (FP8 && !MX && !TOKSCALE) ? (EPI == EPI_SWIGLU ? 2 : (BN + 127) / 128) : 0;
  // the A rows' scales take whole waves (threads 0 .. SAB - 1), the B block
  // scales follow in SA[SAB + q]
  constexpr int SAB = (BM + 63) / 64 * 64;
  static_assert(NQB <= 2 && (NQB == 0 || NTH >= SAB + 64), "a wave past the A rows fetches the B scales");
  const float* __restrict__ sb_base = nullptr;
  int64_t sb_end = 0;
  uint32_t sb_off = 0, sb_step = 0;  // byte offset of this lane's scale at step 0, and per step
  if constexpr (NQB > 0) {
    sb_base = g.b_scale + int64_t(grp) * g.b_scale_gstride;
    sb_end = g.b_scale_gstride * 4;
    const int q = min(lane, NQB - 1);
    const int blk = (EPI == EPI_SWIGLU) ? ((q == 0 ? 0 : g.f) + nt * (BN / 2)) / 128 : n0 / 128 + q;
    sb_off = uint32_t((B_KMAJ ? blk * g.b_scale_ld : blk) * 4);
    sb_step = uint32_t((B_KMAJ ? 1 : g.b_scale_ld) * 4);
  }

  // MXFP8: E8M0 bytes of B (b_scale bytes; group stride b_scale_gstride
  // bytes). K-major B [N, K]: row n's bytes at n * b_scale_ld (= K / 32), so
  // thread tid < BN reads one word per step for tile column tid; K-strided B
  // [K, N]: scale row kb (K block) at kb * b_scale_ld (= N), four bytes per
  // step and column.
  const char* mb_base = nullptr;
  int64_t mb_end = 0;
  int mb_row = 0;  // K-major: byte offset of column tid's scale row
  if constexpr (MX && !TOKMX) {
    mb_base = reinterpret_cast<const char*>(g.b_scale) + int64_t(grp) * g.b_scale_gstride;
    mb_end = B_KMAJ ? int64_t(g.N) * g.b_scale_ld : int64_t(g.K / 32) * g.b_scale_ld;
    if constexpr (B_KMAJ) {
      int grow = n0 + tid;
      if (EPI == EPI_SWIGLU) {  // the B rows' order of the DMA plan above
        const int w = tid / WTN, within = tid % WTN;
        grow = (within / (WTN / 2)) * g.f + nt * (BN / 2) + w * (WTN / 2) + within % (WTN / 2);
      }
      mb_row = grow * g.b_scale_ld;
    }
  }

  // FP8 (row-grouped): the scale word each thread fetches per step, an A-row
  // scale (waves below BM / 64) or a B-block scale (the waves past them):
  // base, range and offsets chosen once here, so that the K loop has no
  // branch on them (a branch splits the loop into several blocks, and the
  // compiler then sinks a step's MFMAs below its wait and barrier)
  const char* sc_base = nullptr;
  int64_t sc_end = 0;
  uint32_t sc_off = 0, sc_inc = 0;
  if constexpr (FP8 && !TOKW) {
    const bool arow = wave < SAB / 64;
    sc_base = arow ? sa_base : reinterpret_cast<const char*>(sb_base);
    sc_end = arow ? sa_end : sb_end;
    sc_off = arow ? uint32_t(tid * g.a_scale_ld * 4) : sb_off;
    sc_inc = arow ? uint32_t((BK / 128) * 4) : sb_step;
  }

  // register-staged operand chunks (K-strided sources) and FP8 row scale
  u32x4 ra[PA::NREG], rb[PB::NREG];
  float rs = 0.0f;
  uint32_t rsb = 0;

  // issue the loads of K step s into stage st: DMA for K-major operands,
  // registers for K-strided ones
  auto issue = [&](ST& st, int s) {
    // steps at or past the end (padding, last prefetch) get empty ranges:
    // for a K-major operand the advanced base would otherwise reach into
    // the next row
    const bool live = s < nk;
    const char* ab = a_base + int64_t(s) * a_step;
    const char* bb = b_base + int64_t(s) * b_step;
    const int64_t an = live ? a_end - int64_t(s) * a_step : 0;
    const int64_t bn = live ? b_end - int64_t(s) * b_step : 0;
    if constexpr (PA::DMA) {
      const u32x4 ar = rsrc_words(ab, an);
#pragma unroll
      for (int j = 0; j < PA::NB; ++j)
        dma16(ar, &st.A[(j * PA::NW + wave) * (1024 / ES)], pa.voff[j]);
    } else {
      const rsrc_t ar = make_rsrc(ab, an);
#pragma unroll
      for (int i = 0; i < 4 * PA::NT; ++i) ra[i] = __builtin_amdgcn_raw_buffer_load_b128(ar, pa.voff[i], 0, 0);
    }
    if constexpr (PB::DMA) {
      const u32x4 br = rsrc_words(bb, bn);
#pragma unroll
      for (int j = 0; j < PB::NB; ++j)
        dma16(br, &st.B[(j * PB::NW + wave) * (1024 / ES)], pb.voff[j]);
    } else {
      const rsrc_t br = make_rsrc(bb, bn);
#pragma unroll
      for (int i = 0; i < 4 * PB::NT; ++i) rb[i] = __builtin_amdgcn_raw_buffer_load_b128(br, pb.voff[i], 0, 0);
    }
    // (the FP8 weight gradients issue through their own loop's issue_t)
    if constexpr (FP8 && !MX && !TOKSCALE && NS > 2) {
      // deep pipelines: the scales land in LDS by DMA like the tiles; wave
      // w < BM / 64 gathers rows 64 w .. 64 w + 63 (rows past the group read
      // 0), the waves past them the B scales
      dma4(rsrc_words(sc_base, live ? sc_end : 0), &st.SA[wave * 64], sc_off + uint32_t(s) * sc_inc);
    } else if constexpr (FP8 && !TOKW) {
      const rsrc_t sr = make_rsrc(sc_base, live ? sc_end : 0);
      rs = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(sr, sc_off + uint32_t(s) * sc_inc, 0, 0));
    }
    if constexpr (MX && !TOKMX) {
      // threads tid < BN (whole waves) fetch a column's word; the others
      // read an empty range (zeros): no branch, as for the FP8 scales
      const rsrc_t sr = make_rsrc(mb_base, (live && wave < BN / 64) ? mb_end : 0);
      if constexpr (B_KMAJ) {
        rsb = __builtin_amdgcn_raw_buffer_load_b32(sr, uint32_t(mb_row + 4 * s), 0, 0);
      } else {
        uint32_t w = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          w |= uint32_t(__builtin_amdgcn_raw_buffer_load_b8(
                   sr, uint32_t((4 * s + q) * g.b_scale_ld + n0 + tid), 0, 0))
               << (8 * q);
        rsb = w;
      }
    }
  };
  // write the register-staged parts of a step into stage st
  auto commit = [&](ST& st) {
    if constexpr (!PA::DMA) {
#pragma unroll
      for (int i = 0; i < PA::NT; ++i) store_transposed<T, BK>(&ra[4 * i], st.A, pa.lrow[i], pa.lk[i]);
    }
    if constexpr (!PB::DMA) {
#pragma unroll
      for (int i = 0; i < PB::NT; ++i) store_transposed<T, BK>(&rb[4 * i], st.B, pb.lrow[i], pb.lk[i]);
    }
    if constexpr (MX && !TOKMX) {
      st.SA[tid] = __builtin_bit_cast(uint32_t, rs);
      st.SB[tid] = rsb;  // entries past BN: zeros, unused
    } else if constexpr (FP8 && !TOKW) {
      st.SA[tid] = rs;
    }
  };

  f32x4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // LM_TDMA fragment: tile columns c0 .. c0 + 16 (one per lane of a 16-lane
  // group), K-rows 32 kk + 8 (lane / 16) .. + 8 from two transpose reads
  auto load_tr = [&](const T* tile, int ROWS, int c0, int kk) {
    typename MF::frag f{};
    if constexpr (sizeof(T) == 2) {
      const int s16 = lane % 16, t = s16 / 4, q = s16 % 4;
      const int kr = kk * 32 + 8 * (lane / 16) + t;
      const int col = c0 + 4 * q;
      const char* p =
          reinterpret_cast<const char*>(tile) + kr * (ROWS * 2) + (((col / 8) ^ tr_swz(kr)) * 16) + (col % 8) * 2;
      const u32x2 lo = lds_read_tr16(p), hi = lds_read_tr16(p + 4 * ROWS * 2);
      f = __builtin_bit_cast(typename MF::frag, u32x4{lo[0], lo[1], hi[0], hi[1]});
    } else if constexpr (sizeof(T) == 1) {
      // K chunks q and q + 4 of the 128-deep block (q = lane / 16), 8 K-rows
      // per transpose read: K-rows 16 q, 16 q + 8, 64 + 16 q, 72 + 16 q
      const int s16 = lane % 16, j = s16 / 2, h = s16 % 2;
      const int col = c0 + 8 * h;
      int w[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kr = 16 * (lane / 16) + 8 * (r & 1) + 64 * (r >> 1) + j;
        const char* p = reinterpret_cast<const char*>(tile) + kr * ROWS +
                        (((col / 16) ^ (ROWS == 256 ? tr8w_swz(kr) : tr8_swz(kr))) * 16) + col % 16;
        const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (__attribute__((address_space(3))) i32x2*)(void*)p);
        w[2 * r] = v[0];
        w[2 * r + 1] = v[1];
      }
      f = i32x8_t{w[0], w[1], w[2], w[3], w[4], w[5], w[6], w[7]};
    }
    return f;
  };
  // fragment i (rows i*16 .. +16 of the wave's A rows) / j (B rows), sub-step kk
  auto load_a = [&](const ST& st, int i, int kk) {
    if constexpr (ALM == LM_TDMA) {
      return load_tr(st.A, BM, wm * WTM + i * 16, kk);
    } else {
      const int r = wm * WTM + i * 16 + (lane % 16), kofs = MF::kofs(lane, kk);
      return MF::load(&st.A[lds_off<T, BK, A_KMAJ>(r, kofs)], &st.A[lds_off<T, BK, A_KMAJ>(r, kofs + MF::K2)]);
    }
  };
  auto load_b = [&](const ST& st, int j, int kk) {
    if constexpr (BLM == LM_TDMA) {
      return load_tr(st.B, BN, wn * WTN + j * 16, kk);
    } else {
      const int r = wn * WTN + j * 16 + (lane % 16), kofs = MF::kofs(lane, kk);
      return MF::load(&st.B[lds_off<T, BK, B_KMAJ>(r, kofs)], &st.B[lds_off<T, BK, B_KMAJ>(r, kofs + MF::K2)]);
    }
  };

  // 8-bit operands: a scheduling barrier right after a step's MFMAs keeps
  // them between the issue of the next step's loads and the wait for them.
  // Left free, the scheduler sinks most of them below the wait and the
  // barrier, and the wait then sits on an idle matrix core (FP8 layer step
  // -1 %, MXFP8 -3 %). bf16 runs about 1 % faster with the compiler's own
  // interleaving, so it keeps it.
  auto pin_mfma = [] {
    if constexpr (sizeof(T) == 1) __builtin_amdgcn_sched_barrier(0);
  };

  // one K step (K block s) on stage st
  auto compute = [&](const ST& st, int s) {
    float sb0 = 0.0f, sb1 = 0.0f;
    if constexpr (NQB > 0) {
      // BK == 128: one scale block per step (a wave's WTN <= 128 columns
      // lie in one 128-column block)
      sb0 = st.SA[SAB + (EPI == EPI_SWIGLU ? 0 : (wn * WTN) / 128)];
      sb1 = st.SA[SAB + (EPI == EPI_SWIGLU ? 1 : (wn * WTN) / 128)];
    }
    if constexpr (MX) {
      // one 128-deep block per step; the matrix core applies the E8M0 byte
      // of K block q = lane / 16 (byte q of the row's or column's word) and
      // accumulates in place
      static_assert(BK == MF::MK, "one MFMA K block per step");
      const int sh = 8 * (lane / 16);
      typename MF::frag bfr[FN], acur, anxt;
      int sbj[FN];
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        bfr[j] = load_b(st, j, 0);
        // (weight gradients: the B words follow the A rows' in SA)
        const uint32_t wj = TOKMX ? st.SA[BM + wn * WTN + j * 16 + lane % 16] : st.SB[wn * WTN + j * 16 + lane % 16];
        sbj[j] = int((wj >> sh) & 0xffu);
      }
      acur = load_a(st, 0, 0);
      static_for<FM>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        if constexpr (i + 1 < FM) anxt = load_a(st, i + 1, 0);
        const int sai = int((st.SA[wm * WTM + i * 16 + lane % 16] >> sh) & 0xffu);
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = MF::mma_scaled(acur, bfr[j], acc[i][j], sai, sbj[j]);
        if constexpr (i + 1 < FM) acur = anxt;
      });
    } else if constexpr (FP8) {
      // one 128-deep block per step: B fragments first, then one A fragment
      // ahead of the FN MFMAs (into temporaries) and their scaled adds
      static_assert(BK == MF::MK, "one MFMA K block per step");
      typename MF::frag bfr[FN], acur, anxt;
      float sbv[FN];  // weight gradients: the scale of each lane's column
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        bfr[j] = load_b(st, j, 0);
        if constexpr (TOKSCALE) sbv[j] = st.SA[BM + wn * WTN + j * 16 + lane % 16];
      }
      acur = load_a(st, 0, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, FN + 1, 0);
      static_for<FM>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        if constexpr (i + 1 < FM) anxt = load_a(st, i + 1, 0);
        const float4 sa4 = *reinterpret_cast<const float4*>(&st.SA[wm * WTM + i * 16 + 4 * (lane / 16)]);
        const float sa[4] = {sa4.x, sa4.y, sa4.z, sa4.w};
        f32x4_t dd[FN];
#pragma unroll
        for (int j = 0; j < FN; ++j) dd[j] = MF::mma(acur, bfr[j], f32x4_t{0.0f, 0.0f, 0.0f, 0.0f});
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const float sbj = TOKSCALE ? sbv[j] : ((EPI == EPI_SWIGLU && j >= FN / 2) ? sb1 : sb0);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(dd[j][r], sa[r] * sbj, acc[i][j][r]);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, (i + 1 < FM) ? 2 : 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, FN, 0);
        if constexpr (i + 1 < FM) acur = anxt;
      });
    } else {
      // Software-pipelined fragment reads: the B fragments of sub-step kk and
      // one A fragment are read ahead of the MFMAs that use them; the order
      // is pinned (one DS read, then FN MFMAs) so that the scheduler does not
      // hoist every read of the next sub-step and run out of registers.
      constexpr int KK = BK / MF::MK;
      typename MF::frag bcur[FN], bnxt[FN], acur, anxt;
#pragma unroll
      for (int j = 0; j < FN; ++j) bcur[j] = load_b(st, j, 0);
      acur = load_a(st, 0, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, FN + 1, 0);
      static_for<KK * FM>([&](auto tc) {
        constexpr int t = decltype(tc)::value;
        constexpr int kk = t / FM, i = t % FM;
        constexpr bool more_a = t + 1 < KK * FM;
        constexpr bool more_b = i == FM - 1 && kk + 1 < KK;
        if constexpr (more_a) anxt = load_a(st, (t + 1) % FM, (t + 1) / FM);
        if constexpr (more_b) {
#pragma unroll
          for (int j = 0; j < FN; ++j) bnxt[j] = load_b(st, j, kk + 1);
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = MF::mma(acur, bcur[j], acc[i][j]);
        constexpr int nreads = (more_a ? 1 : 0) + (more_b ? FN : 0);
        if constexpr (nreads > 0) __builtin_amdgcn_sched_group_barrier(0x100, nreads, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, FN, 0);
        acur = anxt;
        if constexpr (more_b) {
#pragma unroll
          for (int j = 0; j < FN; ++j) bcur[j] = bnxt[j];
        }
      });
    }
  };

  // K loop. Two stages: the loads of step s + 1 are issued before the MFMAs
  // of step s and land (DMA, or registers written to LDS) before the barrier
  // that ends step s; unrolled by two over an even number of steps so that
  // the loop has one exit and no conditional loads (the step past the end
  // of odd step counts and the prefetch past the last step read outside
  // their descriptors' ranges, i.e. zeros, and touch no memory).
  // NS > 2 stages (DMA operands only): the loads of step s + NS - 1 are
  // issued at step s, and the barrier that ends step s waits only for step
  // s + 1 to land, so NS - 1 steps of loads are in flight.
  if constexpr (PERSIST) {
    // Weight gradients. The workgroup runs ntl column tiles of one
    // (group, row block), nk K steps each (a few: the group's rows), as one
    // sequence of Q = ntl * nk steps over the two stages: the loads of step
    // q + 2 go out as soon as every wave is done with step q's stage, across
    // tile boundaries, so that the next tile's loads are in flight while a
    // tile's last step runs and its results are stored. All loads are DMA
    // (NDMA instructions per wave and step: tiles, and FP8 scales); a tile's
    // results go through a staging region of their own, after the next
    // loads have been issued. Loads and stores complete in issue order, so
    // the wait for a step's loads counts the stores issued after them.
    static_assert(NS == 2 && EPI == EPI_STORE && sizeof(TC) == 2, "two stages, plain bf16 stores");
    constexpr int NDMA = PA::NB + PB::NB + (TOKW ? 1 : 0);
    constexpr int EPB = WTN + 8;  // bf16 per staged row (16-byte pad: no bank conflicts)
    constexpr int UPR = WTN / 8;  // 8-column units per staged row
    static_assert(16 * UPR % 64 == 0, "whole store rounds per lane");
    constexpr int EPT = FM * (16 * UPR / 64);  // store instructions per lane and tile
    static_assert(NDMA + 2 * EPT < 64, "vmcnt range");
    __shared__ __attribute__((aligned(16))) bf16_t stg_all[NTH / 64 * 16 * EPB];
    const int ntl = min(max(g.tpw, 1), g.tiles_n - nt);
    const int Q = ntl * nk;
    auto issue_t = [&](ST& st, int q) {
      const int j = q / nk, s = q - j * nk;
      const int64_t jb = int64_t(j) * BN * ES;  // column tile j of the run
      const u32x4 ar = rsrc_words(a_base + int64_t(s) * a_step, a_end - int64_t(s) * a_step);
#pragma unroll
      for (int b = 0; b < PA::NB; ++b) dma16(ar, &st.A[(b * PA::NW + wave) * (1024 / ES)], pa.voff[b]);
      const u32x4 br = rsrc_words(b_base + int64_t(s) * b_step + jb, b_end - int64_t(s) * b_step - jb);
#pragma unroll
      for (int b = 0; b < PB::NB; ++b) dma16(br, &st.B[(b * PB::NW + wave) * (1024 / ES)], pb.voff[b]);
      if constexpr (TOKW) {
        const int64_t so = int64_t(kb0 + s) * ts_ld + (wave * 64 < BM ? 0 : int64_t(j) * BN);
        dma4(rsrc_words(ts_run + so, 256), &st.SA[wave * 64], uint32_t(lane * 4));
      }
    };
    TC* Cb = reinterpret_cast<TC*>(g.C) + int64_t(grp) * g.c_gstride;
    // A lane holds rows 4 (lane / 16) + r, column lane % 16 of each 16 x 16
    // block. Each wave rounds a 16-row block to bf16 into its own staging
    // region and reads it back as 8 consecutive columns per lane, for
    // 16-byte stores; a wave's LDS accesses complete in order, so it needs
    // no barrier. Every lane takes part in every access (no lane-dependent
    // branches around them).
    auto store_tile = [&](int j) {
      bf16_t* stg = stg_all + wave * 16 * EPB;
      const int n0j = n0 + j * BN;
#pragma unroll
      for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int jj = 0; jj < FN; ++jj)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            stg[(4 * (lane / 16) + r) * EPB + jj * 16 + lane % 16] = f32_to_bf16(acc[i][jj][r]);
#pragma unroll
        for (int t = 0; t < 16 * UPR / 64; ++t) {
          const int u = lane + 64 * t;
          const int rr = u / UPR, c8 = u % UPR;
          const uint4 w = *reinterpret_cast<const uint4*>(&stg[rr * EPB + c8 * 8]);
          const int64_t row = m0 + wm * WTM + i * 16 + rr;
          // written once, never read here: streaming stores keep them from
          // displacing the operands in L2
          st_stream(Cb + row * g.ldc + n0j + wn * WTN + c8 * 8, w);
        }
#pragma unroll
        for (int jj = 0; jj < FN; ++jj) acc[i][jj] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      }
    };
    if (Q == 0) {  // no rows: zero gradients
      for (int j = 0; j < ntl; ++j) store_tile(j);
      return;
    }
    issue_t(st0, 0);
    for (int q = 0; q < Q; ++q) {
      ST& cur = (q & 1) ? st1 : st0;
      ST& nxt = (q & 1) ? st0 : st1;
      // issued after step q's loads: the stores of the tile step q - 1 ended
      // (if it ended one)
      if (q >= 1 && q % nk == 0) __builtin_amdgcn_s_waitcnt(vm_wait(EPT));
      else wait_vm0();
      // every wave's loads of step q landed, and every wave is done with
      // step q - 1's stage
      __syncthreads();
      if (q + 1 < Q) issue_t(nxt, q + 1);
      __builtin_amdgcn_sched_barrier(0);
      compute(cur, 0);
      pin_mfma();
      if ((q + 1) % nk == 0) store_tile(q / nk);
    }
    return;
  } else if constexpr (NS == 2) {
    if (nk > 0) {
      const int nk2 = (nk + 1) & ~1;
      issue(st0, 0);
      commit(st0);
      wait_vm0();
      __syncthreads();
      for (int s = 0; s < nk2; s += 2) {
        issue(st1, s + 1);
        __builtin_amdgcn_sched_barrier(0);
        compute(st0, s);
        pin_mfma();
        commit(st1);
        wait_vm0();
        __syncthreads();
        issue(st0, s + 2);
        __builtin_amdgcn_sched_barrier(0);
        compute(st1, s + 1);
        pin_mfma();
        commit(st0);
        wait_vm0();
        __syncthreads();
      }
    }
  } else {
    static_assert(PA::DMA && PB::DMA && (!FP8 || (!MX && !TOKSCALE && NTH / 64 * 64 >= BM)),
                  "deep pipelines take DMA operands (and FP8 row scales) only");
    // DMA instructions per wave and step (FP8: one more, the row scales)
    constexpr int NDMA = PA::NB + PB::NB + (FP8 ? 1 : 0);
    constexpr int LEFT = NDMA * (NS - 2);  // may stay in flight at a step's end
    static_assert(LEFT < 64, "vmcnt range");
    constexpr int WAIT = (LEFT & 15) | ((LEFT >> 4) << 14) | (7 << 4) | (15 << 8);
    if (nk > 0) {
#pragma unroll
      for (int p = 0; p < NS - 1; ++p) issue(stv[p], p);
      __builtin_amdgcn_s_waitcnt(WAIT);
      __syncthreads();
      for (int s = 0; s < nk; ++s) {
        issue(stv[(s + NS - 1) % NS], s + NS - 1);
        __builtin_amdgcn_sched_barrier(0);
        compute(stv[s % NS], s);
        pin_mfma();
        __builtin_amdgcn_s_waitcnt(WAIT);
        __syncthreads();
      }
      // the last prefetches (zeros) may still be landing: the epilogue
      // reuses their LDS
      wait_vm0();
      __syncthreads();
    }
  }

  // Epilogue through LDS (all stages are free after the K loop's last
  // barrier). A lane holds rows 4 (lane / 16) + r, column lane % 16 of each
  // 16 x 16 accumulator block; every wave writes one 16-row block of its
  // tile at a time to a private LDS region and reads it back as 8
  // consecutive columns per lane, so that global loads and stores are 16
  // bytes wide. A wave's LDS accesses complete in order, so no barrier is
  // needed between its writes and reads.
  constexpr int EP = WTN + 4;          // floats per staged row (pad: no bank conflicts)
  constexpr int UPR = WTN / 8;         // 8-column units per staged row
  static_assert(int(sizeof(ST)) * NS >= NTH / 64 * 16 * EP * 4, "staging fits in the LDS stages");
  float* stg = reinterpret_cast<float*>(stv) + wave * 16 * EP;
  TC* Cb = reinterpret_cast<TC*>(g.C);
  if (MODE == G_KSPLIT) Cb += int64_t(grp) * g.c_gstride;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) stg[(4 * (lane / 16) + r) * EP + j * 16 + lane % 16] = acc[i][j][r];
    const int rbase = wm * WTM + i * 16;  // tile row of the block's first row
    if constexpr (EPI == EPI_SWIGLU) {
      // staged columns [0, WTN/2) are gate values, [WTN/2, WTN) up values
      // of the same output columns
      TO* GU = reinterpret_cast<TO*>(g.aux0);
      TO* H = reinterpret_cast<TO*>(g.aux1);
#pragma unroll
      for (int u = lane; u < 16 * UPR / 2; u += 64) {
        const int rr = u / (UPR / 2), c8 = u % (UPR / 2);
        const int rl = rbase + rr;
        if (rl < mrows) {
          const int64_t row = row0 + rl;
          const int col = nt * (BN / 2) + wn * (WTN / 2) + c8 * 8;
          float G[8], U[8], Hv[8];
          lds_read8(&stg[rr * EP + c8 * 8], G);
          lds_read8(&stg[rr * EP + WTN / 2 + c8 * 8], U);
          round8<TO>(G);
          round8<TO>(U);
#pragma unroll
          for (int e = 0; e < 8; ++e) Hv[e] = swiglu_h(G[e], U[e]);
          if (GU) {
            store8<TO>(GU + row * (2 * g.f) + col, G);
            store8<TO>(GU + row * (2 * g.f) + g.f + col, U);
          }
          store8<TO>(H + row * g.f + col, Hv);
        }
      }
    } else {
#pragma unroll
      for (int u = lane; u < 16 * UPR; u += 64) {
        const int rr = u / UPR, c8 = u % UPR;
        const int rl = rbase + rr;
        if (MODE == G_KSPLIT || rl < mrows) {
          const int64_t row = (MODE == G_ROWS) ? int64_t(row0 + rl) : int64_t(m0 + rl);
          const int col = n0 + wn * WTN + c8 * 8;
          float v[8];
          lds_read8(&stg[rr * EP + c8 * 8], v);
          if constexpr (EPI == EPI_STORE && MODE == G_KSPLIT) {
            // weight gradients: written once, never read by this kernel;
            // streaming stores keep them from displacing the operands in L2
            store8_stream<TC>(Cb + row * g.ldc + col, v);
          } else if constexpr (EPI == EPI_STORE) {
            store8<TC>(Cb + row * g.ldc + col, v);
          } else {  // EPI_DSWIGLU: v = dH; C = dGU [rows, 2f]
            const TO* GU = reinterpret_cast<const TO*>(g.aux0);
            TO* D = reinterpret_cast<TO*>(g.C);
            float G[8], U[8], dG[8], dU[8];
            load8<TO>(GU + row * (2 * g.f) + col, G);
            load8<TO>(GU + row * (2 * g.f) + g.f + col, U);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float sg = 1.0f / (1.0f + expf(-G[e]));
              dG[e] = v[e] * U[e] * sg * (1.0f + G[e] * (1.0f - sg));
              dU[e] = v[e] * G[e] * sg;
            }
            store8<TO>(D + row * (2 * g.f) + col, dG);
            store8<TO>(D + row * (2 * g.f) + g.f + col, dU);
            if (g.aux1) {  // activation recompute: H for the weight gradient
              float Hv[8];
#pragma unroll
              for (int e = 0; e < 8; ++e) Hv[e] = swiglu_h(G[e], U[e]);
              store8<TO>(reinterpret_cast<TO*>(g.aux1) + row * g.f + col, Hv);
            }
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// FP8 row quantisation (1 x 128 blocks), 16 lanes per block
// ---------------------------------------------------------------------------
template <typename TS>
__global__ __launch_bounds__(256) void quant_rows_kernel(const TS* __restrict__ src, fp8_t* __restrict__ q,
                                                         float* __restrict__ scale, int64_t nchunks) {
  constexpr int V = 8;  // elements per lane
  const int64_t ch = blockIdx.x * int64_t(256) + threadIdx.x;  // chunk of 8 elements
  const bool ok = ch < nchunks;
  float v[V];
  if (ok) {
    if constexpr (sizeof(TS) == 2) {
      Vec16<bf16_t>::load(reinterpret_cast<const bf16_t*>(src) + ch * V, v);
    } else {
      Vec16<float>::load(reinterpret_cast<const float*>(src) + ch * V, v);
      Vec16<float>::load(reinterpret_cast<const float*>(src) + ch * V + 4, v + 4);
    }
  } else {
    for (int i = 0; i < V; ++i) v[i] = 0.0f;
  }
  float amax = 0.0f;
  for (int i = 0; i < V; ++i) amax = fmaxf(amax, fabsf(v[i]));
  for (int o = 8; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, kWave));
  const float s = (amax == 0.0f) ? 1.0f : amax / 448.0f;
  const u32x2 w = fp8_encode8(v, s, 1.0f / s, fp8_fast_scale(s));
  if (ok) {
    *reinterpret_cast<u32x2*>(q + ch * V) = w;
    if ((ch & 15) == 0) scale[ch / 16] = s;  // rows are whole 128-blocks
  }
}

void launch_quant_rows(const void* src, bool src_bf16, int64_t rows, int64_t cols, uint8_t* q, float* scale,
                       hipStream_t st) {
  const int64_t nchunks = rows * cols / 8;
  const int64_t grid = (nchunks + 255) / 256;
  if (grid <= 0) return;
  if (src_bf16)
    quant_rows_kernel<bf16_t><<<grid, 256, 0, st>>>(reinterpret_cast<const bf16_t*>(src), q, scale, nchunks);
  else
    quant_rows_kernel<float><<<grid, 256, 0, st>>>(reinterpret_cast<const float*>(src), q, scale, nchunks);
}

// ---------------------------------------------------------------------------
// MXFP8 quantisation: E4M3 codes of v * 2^-x with one E8M0 byte x + 127 per
// block of 32 (x = mx_scale_exp of the block's largest magnitude, so that no
// scaled value exceeds 448; ldexp is an exact rescaling, then round to
// nearest even by v_cvt_pk_fp8_f32). Row blocks (1 x 32): 4 lanes per block;
// column blocks (32 x 1): one thread per block, 32 rows apart.
// ---------------------------------------------------------------------------
template <typename TS>
__device__ __forceinline__ void load8_src(const TS* src, int64_t i, float* v) {
  if constexpr (sizeof(TS) == 2) {
    Vec16<bf16_t>::load(reinterpret_cast<const bf16_t*>(src) + i, v);
  } else {
    Vec16<float>::load(reinterpret_cast<const float*>(src) + i, v);
    Vec16<float>::load(reinterpret_cast<const float*>(src) + i + 4, v + 4);
  }
}


template <typename TS>
__global__ __launch_bounds__(256) void quant_mx_rows_kernel(const TS* __restrict__ src, uint8_t* __restrict__ q,
                                                            uint8_t* __restrict__ e8m0, int64_t nchunks) {
  const int64_t ch = blockIdx.x * int64_t(256) + threadIdx.x;  // chunk of 8 elements
  const bool ok = ch < nchunks;
  float v[8];
  if (ok) load8_src(src, ch * 8, v);
  else
    for (int i = 0; i < 8; ++i) v[i] = 0.0f;
  float amax = 0.0f;
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  for (int o = 2; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, kWave));
  const int x = mx_scale_exp(amax);
  const u32x2 c = mx_codes8(v, x);
  if (ok) {
    *reinterpret_cast<u32x2*>(q + ch * 8) = c;
    if ((ch & 3) == 0) e8m0[ch / 4] = uint8_t(x + 127);  // rows are whole 32-blocks
  }
}

template <typename TS>
__global__ __launch_bounds__(256) void quant_mx_cols_kernel(const TS* __restrict__ src, uint8_t* __restrict__ q,
                                                            uint8_t* __restrict__ e8m0, int64_t C,
                                                            int64_t col_blocks) {
  const int64_t br = blockIdx.x / col_blocks;  // block row: rows 32 br .. + 32
  const int64_t c = (blockIdx.x % col_blocks) * 256 + threadIdx.x;
  if (c >= C) return;
  const TS* p = src + br * 32 * C + c;
  float v[32];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    if constexpr (sizeof(TS) == 2) v[i] = bf16_to_f32(reinterpret_cast<const bf16_t*>(p)[int64_t(i) * C]);
    else v[i] = reinterpret_cast<const float*>(p)[int64_t(i) * C];
    amax = fmaxf(amax, fabsf(v[i]));
  }
  const int x = mx_scale_exp(amax);
#pragma unroll
  for (int i = 0; i < 32; i += 8) {
    const u32x2 w = mx_codes8(v + i, x);
#pragma unroll
    for (int b = 0; b < 8; ++b) q[(br * 32 + i + b) * C + c] = uint8_t(w[b / 4] >> (8 * (b % 4)));
  }
  e8m0[br * C + c] = uint8_t(x + 127);
}

void launch_quant_mx_rows(const void* src, bool src_bf16, int64_t rows, int64_t cols, uint8_t* q,
                          uint8_t* e8m0, hipStream_t st) {
  const int64_t nchunks = rows * cols / 8;
  const int64_t grid = (nchunks + 255) / 256;
  if (grid <= 0) return;
  if (src_bf16)
    quant_mx_rows_kernel<bf16_t><<<grid, 256, 0, st>>>(reinterpret_cast<const bf16_t*>(src), q, e8m0, nchunks);
  else
    quant_mx_rows_kernel<float><<<grid, 256, 0, st>>>(reinterpret_cast<const float*>(src), q, e8m0, nchunks);
}

void launch_quant_mx_cols(const void* src, bool src_bf16, int64_t rows, int64_t cols, uint8_t* q,
                          uint8_t* e8m0, hipStream_t st) {
  const int64_t cb = (cols + 255) / 256;
  const int64_t grid = (rows / 32) * cb;
  if (grid <= 0) return;
  if (src_bf16)
    quant_mx_cols_kernel<bf16_t><<<grid, 256, 0, st>>>(reinterpret_cast<const bf16_t*>(src), q, e8m0, cols, cb);
  else
    quant_mx_cols_kernel<float><<<grid, 256, 0, st>>>(reinterpret_cast<const float*>(src), q, e8m0, cols, cb);
}

// ---------------------------------------------------------------------------
// FP8 weight-gradient operands: E4M3 in blocks of 128 consecutive rows x 1
// column inside each expert's rows (the contraction of dW = P^T Q runs over
// the expert's rows), one fp32 scale amax / 448 per block and column. Block
// b of the concatenated block list is block b - kblk[e] of expert e, where
// kblk[e] = sum of ceil(rows / 128) over the experts before e.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void kblock_offsets_kernel(const int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ kblk, int G) {
  __shared__ int s_wave[16];
  const int g = threadIdx.x;
  const int c = g < G ? (offsets[g + 1] - offsets[g] + 127) / 128 : 0;
  int v = c;
  const int lane = lane_id();
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o, kWave);
    if (lane >= o) v += u;
  }
  if (lane == 63) s_wave[g / kWave] = v;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < g / kWave; ++w) before += s_wave[w];
  if (g < G) kblk[g + 1] = before + v;
  if (g == 0) kblk[0] = 0;
}

// One workgroup per (block, 128 columns): thread (cg, rg) holds columns
// 8 cg .. 8 cg + 7 of rows rg, rg + 16, ..., rg + 112 of the block in
// registers; the column maxima meet in LDS, where 128 threads turn them into
// the column scales and their reciprocals once (a division each), for every
// thread to read. Sources: bf16 rows (E4M3 sources take
// quant_tokens_f8src_kernel). ROWQ: the same read also quantises each row's
// 128 columns as one 1 x 128 block (the data-gradient products' operand),
// into rq / rs [A, C/128]. The 16 threads holding rows rg + 16 i (one 16-lane
// group of a wave) reduce their 8 row maxima by a transposing butterfly:
// each exchange step halves the rows a lane keeps, so after four steps lane
// cg holds the whole maximum of row cg / 2, divides once, and the row scales
// go back to the group by lane broadcasts.
template <bool ROWQ>
__global__ __launch_bounds__(256) void quant_tokens_kernel(const bf16_t* __restrict__ src,
                                                           const int32_t* __restrict__ offsets,
                                                           const int32_t* __restrict__ kblk, int G,
                                                           int64_t C, fp8_t* __restrict__ q,
                                                           float* __restrict__ scale, fp8_t* __restrict__ rq,
                                                           float* __restrict__ rs) {
  __shared__ float s_max[16][129];
  __shared__ float s_sc[128], s_rc[128];
  __shared__ int s_fast[128];
  const int b = blockIdx.x;
  if (b >= kblk[G]) return;
  // the expert owning block b: the last e with kblk[e] <= b
  int lo = 0, hi = G - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (kblk[mid] <= b) lo = mid;
    else hi = mid - 1;
  }
  const int64_t r0 = int64_t(offsets[lo]) + int64_t(b - kblk[lo]) * 128;
  const int nrows = int(min(int64_t(128), int64_t(offsets[lo + 1]) - r0));
  const int cg = threadIdx.x % 16, rg = threadIdx.x / 16;
  const int64_t c0 = int64_t(blockIdx.y) * 128 + cg * 8;  // C is a multiple of 128
  // All 8 row loads go out together: a row past the block reads the
  // block's last row (nrows >= 1, so in bounds) and is zeroed after. (Under
  // a per-row branch each load waited for its data before the next one.)
  uint4 raw[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    raw[i] = *reinterpret_cast<const uint4*>(src + (r0 + min(rg + 16 * i, nrows - 1)) * C + c0);
  float v[8][8];
  float m[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) m[c] = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    Vec16<bf16_t>::unpack(raw[i], v[i]);
    const bool in = rg + 16 * i < nrows;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      v[i][c] = in ? v[i][c] : 0.0f;
      m[c] = fmaxf(m[c], fabsf(v[i][c]));
    }
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) s_max[rg][cg * 8 + c] = m[c];
  if constexpr (ROWQ) {
    // 1 x 128 row blocks: this lane's part of the 8 row maxima
    float x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[i] = 0.0f;
#pragma unroll
      for (int c = 0; c < 8; ++c) x[i] = fmaxf(x[i], fabsf(v[i][c]));
    }
    // transposing butterfly over the 16 lanes of the row group: at the step
    // over lane bit h, a lane keeps the half of its rows selected by that
    // bit and takes its partner's values for them
    const int b3 = (cg >> 3) & 1, b2 = (cg >> 2) & 1, b1 = (cg >> 1) & 1;
    float y[4], z[2];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      y[j] = fmaxf(b3 ? x[j + 4] : x[j], __shfl_xor(b3 ? x[j] : x[j + 4], 8, kWave));
#pragma unroll
    for (int j = 0; j < 2; ++j)
      z[j] = fmaxf(b2 ? y[j + 2] : y[j], __shfl_xor(b2 ? y[j] : y[j + 2], 4, kWave));
    float a = fmaxf(b1 ? z[1] : z[0], __shfl_xor(b1 ? z[0] : z[1], 2, kWave));
    a = fmaxf(a, __shfl_xor(a, 1, kWave));  // the maximum of row 4 b3 + 2 b2 + b1 = cg / 2
    const float sr_own = (a == 0.0f) ? 1.0f : a / 448.0f;
    const float rr_own = 1.0f / sr_own;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int rr = rg + 16 * i;
      const float sr = __shfl(sr_own, 2 * i, 16), rsr = __shfl(rr_own, 2 * i, 16);
      if (rr < nrows) {
        *reinterpret_cast<u32x2*>(rq + (r0 + rr) * C + c0) = fp8_encode8(v[i], sr, rsr, fp8_fast_scale(sr));
        if (cg == 0) rs[(r0 + rr) * (C / 128) + c0 / 128] = sr;
      }
    }
  }
  __syncthreads();
  if (threadIdx.x < 128) {  // waves 0 and 1: one column each
    const int col = threadIdx.x;
    float a = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) a = fmaxf(a, s_max[r][col]);
    const float scol = (a == 0.0f) ? 1.0f : a / 448.0f;
    s_sc[col] = scol;
    s_rc[col] = 1.0f / scol;
    s_fast[col] = fp8_fast_scale(scol) ? 1 : 0;
  }
  __syncthreads();
  float sc[8], rc[8];
  bool fast = true;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    sc[c] = s_sc[cg * 8 + c];
    rc[c] = s_rc[cg * 8 + c];
    fast = fast && s_fast[cg * 8 + c] != 0;
  }
  if (rg == 0) {
    float* sp = scale + int64_t(b) * C + c0;
    *reinterpret_cast<float4*>(sp) = float4{sc[0], sc[1], sc[2], sc[3]};
    *reinterpret_cast<float4*>(sp + 4) = float4{sc[4], sc[5], sc[6], sc[7]};
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int rr = rg + 16 * i;
    if (rr < nrows) *reinterpret_cast<u32x2*>(q + (r0 + rr) * C + c0) = fp8_encode8(v[i], sc, rc, fast);
  }
}

// The same blocks from E4M3 sources (X and H, with fp32 scales per 1 x 128
// block of a row), with 16-byte accesses: thread (cg, rg) holds columns
// 16 cg .. 16 cg + 15 of rows rg, rg + 32, rg + 64, rg + 96 of the block;
// the column maxima meet in LDS, where 128 threads turn them into the scales
// and reciprocals. The arithmetic is quant_tokens_kernel's.
__global__ __launch_bounds__(256) void quant_tokens_f8src_kernel(const fp8_t* __restrict__ src,
                                                                 const float* __restrict__ src_scale,
                                                                 const int32_t* __restrict__ offsets,
                                                                 const int32_t* __restrict__ kblk, int G, int64_t C,
                                                                 fp8_t* __restrict__ q, float* __restrict__ scale) {
  __shared__ __attribute__((aligned(16))) float s_max[32][132];  // 16-byte rows: float4 stores
  __shared__ __attribute__((aligned(16))) float s_sc[128];
  __shared__ __attribute__((aligned(16))) float s_rc[128];
  __shared__ int s_fast[128];
  const int b = blockIdx.x;
  if (b >= kblk[G]) return;
  int lo = 0, hi = G - 1;  // the expert owning block b: the last e with kblk[e] <= b
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (kblk[mid] <= b) lo = mid;
    else hi = mid - 1;
  }
  const int64_t r0 = int64_t(offsets[lo]) + int64_t(b - kblk[lo]) * 128;
  const int nrows = int(min(int64_t(128), int64_t(offsets[lo + 1]) - r0));
  const int cg = threadIdx.x % 8, rg = threadIdx.x / 8;
  const int64_t c0 = int64_t(blockIdx.y) * 128 + cg * 16;  // C is a multiple of 128
  // all 4 row loads (codes and scale) go out together: a row past the
  // block reads the block's last row (in bounds) and is zeroed after
  u32x4 raw[4];
  float rsc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t r = r0 + min(rg + 32 * i, nrows - 1);
    raw[i] = *reinterpret_cast<const u32x4*>(src + r * C + c0);
    rsc[i] = src_scale[r * (C / 128) + blockIdx.y];
  }
  float v[4][16];
  float m[16];
#pragma unroll
  for (int c = 0; c < 16; ++c) m[c] = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bool in = rg + 32 * i < nrows;
    const u32x4 w = raw[i];
    const float sc = rsc[i];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[i][4 * k] = __builtin_amdgcn_cvt_f32_fp8(w[k], 0) * sc;
      v[i][4 * k + 1] = __builtin_amdgcn_cvt_f32_fp8(w[k], 1) * sc;
      v[i][4 * k + 2] = __builtin_amdgcn_cvt_f32_fp8(w[k], 2) * sc;
      v[i][4 * k + 3] = __builtin_amdgcn_cvt_f32_fp8(w[k], 3) * sc;
    }
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      v[i][c] = in ? v[i][c] : 0.0f;
      m[c] = fmaxf(m[c], fabsf(v[i][c]));
    }
  }
#pragma unroll
  for (int c = 0; c < 16; c += 4)
    *reinterpret_cast<float4*>(&s_max[rg][cg * 16 + c]) = float4{m[c], m[c + 1], m[c + 2], m[c + 3]};
  __syncthreads();
  if (threadIdx.x < 128) {  // waves 0 and 1: one column each
    const int col = threadIdx.x;
    float a = 0.0f;
#pragma unroll
    for (int r = 0; r < 32; ++r) a = fmaxf(a, s_max[r][col]);
    const float scol = (a == 0.0f) ? 1.0f : a / 448.0f;
    s_sc[col] = scol;
    s_rc[col] = 1.0f / scol;
    s_fast[col] = fp8_fast_scale(scol) ? 1 : 0;
    scale[int64_t(b) * C + int64_t(blockIdx.y) * 128 + col] = scol;
  }
  __syncthreads();
  float sc[16], rc[16];
  bool fast = true;
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    sc[c] = s_sc[cg * 16 + c];
    rc[c] = s_rc[cg * 16 + c];
    fast = fast && s_fast[cg * 16 + c] != 0;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rr = rg + 32 * i;
    const u32x2 lo8 = fp8_encode8(v[i], sc, rc, fast);
    const u32x2 hi8 = fp8_encode8(v[i] + 8, sc + 8, rc + 8, fast);
    if (rr < nrows) *reinterpret_cast<u32x4*>(q + (r0 + rr) * C + c0) = u32x4{lo8[0], lo8[1], hi8[0], hi8[1]};
  }
}

static int64_t token_blocks_bound(int64_t A, int64_t G) { return (A + G * 127) / 128; }

// MXFP8 weight-gradient operands: E4M3 in blocks of 32 consecutive rows x 1
// column inside each expert's rows, one E8M0 byte per block (the MXFP8 rule
// of the row quantiser). The four blocks of a 128-row block and column share
// one word, byte q for rows 32 q .. 32 q + 31 of the 128-row block: the
// per-K-step scale word of the weight-gradient GEMM. Rows past the expert's
// end count as zeros (their blocks take byte 127). Block b of the
// concatenated 128-row block list is block b - kblk[e] of expert e. One
// workgroup per (128-row block, 128 columns), thread (cg, rg) holding
// columns 8 cg .. 8 cg + 7 of rows rg, rg + 16, ..., rg + 112 (rows rg + 16 i
// lie in 32-row block i / 2); the block maxima meet in LDS. Sources: bf16
// rows, or E4M3 codes with one E8M0 byte per 1 x 32 block of a row, taken as
// code x 2^(byte - 127) in fp32. ROWQ (bf16 sources): the same read also
// quantises each row in 1 x 32 blocks (the data-gradient products'
// operand, exactly as the row quantiser does), into rq [A, C] and re8m0
// [A, C/32]: the four threads of a block (lanes 4 j .. 4 j + 3 of a 16-lane
// group) reduce its amax with lane shuffles.
template <bool SRC_MX, bool ROWQ>
__global__ __launch_bounds__(256) void quant_tokens_mx_kernel(const void* __restrict__ src,
                                                              const uint8_t* __restrict__ src_e8m0,
                                                              const int32_t* __restrict__ offsets,
                                                              const int32_t* __restrict__ kblk, int G, int64_t C,
                                                              fp8_t* __restrict__ q, uint32_t* __restrict__ words,
                                                              fp8_t* __restrict__ rq, uint8_t* __restrict__ re8m0) {
  static_assert(!(SRC_MX && ROWQ), "row blocks are taken from bf16 sources");
  __shared__ __attribute__((aligned(16))) float s_max[16][4][132];  // 16-byte rows: float4 stores
  __shared__ int s_x[4][128];
  const int b = blockIdx.x;
  if (b >= kblk[G]) return;
  int lo = 0, hi = G - 1;  // the expert owning block b: the last e with kblk[e] <= b
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (kblk[mid] <= b) lo = mid;
    else hi = mid - 1;
  }
  const int64_t r0 = int64_t(offsets[lo]) + int64_t(b - kblk[lo]) * 128;
  const int nrows = int(min(int64_t(128), int64_t(offsets[lo + 1]) - r0));
  const int cg = threadIdx.x % 16, rg = threadIdx.x / 16;
  const int64_t c0 = int64_t(blockIdx.y) * 128 + cg * 8;  // C is a multiple of 128
  // All 8 row loads go out together: a row past the block reads the
  // block's last row (nrows >= 1, so in bounds) and is zeroed after. (Under
  // a per-row branch each load waited for its data before the next one.)
  float v[8][8];
  if constexpr (SRC_MX) {
    u32x2 raw[8];
    int rx[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t r = r0 + min(rg + 16 * i, nrows - 1);
      raw[i] = *reinterpret_cast<const u32x2*>(static_cast<const fp8_t*>(src) + r * C + c0);
      rx[i] = int(src_e8m0[r * (C / 32) + c0 / 32]);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const u32x2 w = raw[i];
      const int x = rx[i] - 127;
      const float f8[8] = {__builtin_amdgcn_cvt_f32_fp8(w[0], 0), __builtin_amdgcn_cvt_f32_fp8(w[0], 1),
                           __builtin_amdgcn_cvt_f32_fp8(w[0], 2), __builtin_amdgcn_cvt_f32_fp8(w[0], 3),
                           __builtin_amdgcn_cvt_f32_fp8(w[1], 0), __builtin_amdgcn_cvt_f32_fp8(w[1], 1),
                           __builtin_amdgcn_cvt_f32_fp8(w[1], 2), __builtin_amdgcn_cvt_f32_fp8(w[1], 3)};
      const bool in = rg + 16 * i < nrows;
#pragma unroll
      for (int c = 0; c < 8; ++c) v[i][c] = in ? ldexpf(f8[c], x) : 0.0f;
    }
  } else {
    uint4 raw[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      raw[i] = *reinterpret_cast<const uint4*>(static_cast<const bf16_t*>(src) +
                                               (r0 + min(rg + 16 * i, nrows - 1)) * C + c0);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      Vec16<bf16_t>::unpack(raw[i], v[i]);
      const bool in = rg + 16 * i < nrows;
#pragma unroll
      for (int c = 0; c < 8; ++c) v[i][c] = in ? v[i][c] : 0.0f;
    }
  }
  if constexpr (ROWQ) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int rr = rg + 16 * i;
      float a = 0.0f;
#pragma unroll
      for (int c = 0; c < 8; ++c) a = fmaxf(a, fabsf(v[i][c]));
      a = fmaxf(a, __shfl_xor(a, 1, kWave));
      a = fmaxf(a, __shfl_xor(a, 2, kWave));
      const int x = mx_scale_exp(a);
      if (rr < nrows) {
        *reinterpret_cast<u32x2*>(rq + (r0 + rr) * C + c0) = mx_codes8(v[i], x);
        if ((cg & 3) == 0) re8m0[(r0 + rr) * (C / 32) + c0 / 32] = uint8_t(x + 127);
      }
    }
  }
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) {
    float m[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) m[c] = fmaxf(fabsf(v[2 * qb][c]), fabsf(v[2 * qb + 1][c]));
    *reinterpret_cast<float4*>(&s_max[rg][qb][cg * 8]) = float4{m[0], m[1], m[2], m[3]};
    *reinterpret_cast<float4*>(&s_max[rg][qb][cg * 8 + 4]) = float4{m[4], m[5], m[6], m[7]};
  }
  __syncthreads();
  {  // 512 (32-row block, column) pairs, two per thread
    const int col = threadIdx.x % 128, q0 = (threadIdx.x / 128) * 2;
#pragma unroll
    for (int qb = q0; qb < q0 + 2; ++qb) {
      float a = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) a = fmaxf(a, s_max[r][qb][col]);
      s_x[qb][col] = mx_scale_exp(a);
    }
  }
  __syncthreads();
  if (threadIdx.x < 128) {
    const int col = threadIdx.x;
    uint32_t w = 0;
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) w |= uint32_t(s_x[qb][col] + 127) << (8 * qb);
    words[int64_t(b) * C + int64_t(blockIdx.y) * 128 + col] = w;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int rr = rg + 16 * i;
    int x[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) x[c] = s_x[i / 2][cg * 8 + c];
    if (rr < nrows) *reinterpret_cast<u32x2*>(q + (r0 + rr) * C + c0) = mx_codes8(v[i], x);
  }
}

// src [A, C] (bf16, or E4M3 codes with [A, C/32] E8M0 row-block bytes) ->
// q [A, C] E4M3 and words [token_blocks_bound(A, G), C] (rows past the
// actual block count are not written); with rq (bf16 sources) also the
// 1 x 32 row blocks rq [A, C], re8m0 [A, C/32] from the same read
static void quant_tokens_mx(const void* src, const uint8_t* src_e8m0, const int32_t* offsets, const int32_t* kblk,
                            int64_t G, int64_t A, int64_t C, fp8_t* q, uint32_t* words, hipStream_t st,
                            fp8_t* rq = nullptr, uint8_t* re8m0 = nullptr) {
  const dim3 grid(unsigned(token_blocks_bound(A, G)), unsigned(C / 128));
  if (grid.x == 0) return;
  if (src_e8m0)
    quant_tokens_mx_kernel<true, false><<<grid, 256, 0, st>>>(src, src_e8m0, offsets, kblk, int(G), C, q, words,
                                                             nullptr, nullptr);
  else if (rq)
    quant_tokens_mx_kernel<false, true><<<grid, 256, 0, st>>>(src, nullptr, offsets, kblk, int(G), C, q, words, rq,
                                                             re8m0);
  else
    quant_tokens_mx_kernel<false, false><<<grid, 256, 0, st>>>(src, nullptr, offsets, kblk, int(G), C, q, words,
                                                              nullptr, nullptr);
}

// src [A, C] (bf16, or E4M3 codes with [A, C/128] fp32 row-block scales)
// -> q [A, C] E4M3 and scale [token_blocks_bound(A, G), C] (rows past the
// actual block count are not written); with rq (bf16 sources) also the
// 1 x 128 row blocks rq [A, C], rs [A, C/128] from the same read
static void quant_tokens(const void* src, const float* src_scale, const int32_t* offsets,
                         const int32_t* kblk, int64_t G, int64_t A, int64_t C, fp8_t* q, float* scale,
                         hipStream_t st, fp8_t* rq = nullptr, float* rs = nullptr) {
  const dim3 grid(unsigned(token_blocks_bound(A, G)), unsigned(C / 128));
  if (grid.x == 0) return;
  if (src_scale)
    quant_tokens_f8src_kernel<<<grid, 256, 0, st>>>(static_cast<const fp8_t*>(src), src_scale, offsets, kblk,
                                                    int(G), C, q, scale);
  else if (rq)
    quant_tokens_kernel<true><<<grid, 256, 0, st>>>(static_cast<const bf16_t*>(src), offsets, kblk, int(G), C, q,
                                                    scale, rq, rs);
  else
    quant_tokens_kernel<false><<<grid, 256, 0, st>>>(static_cast<const bf16_t*>(src), offsets, kblk, int(G), C, q,
                                                     scale, nullptr, nullptr);
}

// ---------------------------------------------------------------------------
// Tile configurations: BM x BN output tile, BK deep, WM x WN waves, NS LDS
// stages.
//   Small: 128 x 128, 4 waves of 64 x 64, 2 stages of 32 KB (every dtype;
//          two workgroups per CU hide each other's load latency)
//   Big:   256 x 256, 8 waves of 128 x 64, 2 stages of 64 KB: half the
//          operand bytes per flop of Small and a quarter of the tiles
//   Wgrad: 128 x 256, 4 waves of 64 x 128, 3 stages of 24 KB (BK = 32)
//          for the weight gradients, whose K (an expert's rows) is often
//          short: two workgroups per CU, so one's prologue and epilogue run
//          under the other's MFMAs (measured against Big's tile with 4
//          stages: Qwen3-style skewed experts 1.23 -> 0.91 ms per launch,
//          Mixtral- and DeepSeek-style layers unchanged)
template <typename T, int BM_, int BN_, int BK_, int WM_, int WN_, int NS_>
struct Cfg {
  typedef T type;
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_, NS = NS_;
};
template <typename T> struct SmallCfg;
template <> struct SmallCfg<bf16_t> : Cfg<bf16_t, 128, 128, 64, 2, 2, 2> {};
template <> struct SmallCfg<float> : Cfg<float, 128, 128, 32, 2, 2, 2> {};
template <> struct SmallCfg<fp8_t> : Cfg<fp8_t, 128, 128, 128, 2, 2, 2> {};
template <> struct SmallCfg<mx8_t> : Cfg<mx8_t, 128, 128, 128, 2, 2, 2> {};
// FP8 / MXFP8 160 x 128 tile (4 waves of 80 x 64, two 37 KB stages, two
// workgroups per CU) for experts of 129 to 320 rows on average: two row
// tiles cover up to 320 rows where the 128-row tile needs three, the last
// often a few rows that still stream the whole weight panel
template <typename T> using MidCfg8 = Cfg<T, 160, 128, 128, 2, 2, 2>;
// bf16 160 x 128 tile (BK 64, two 36 KB stages), for the same experts
typedef Cfg<bf16_t, 160, 128, 64, 2, 2, 2> MidCfg16;
typedef Cfg<bf16_t, 256, 256, 64, 2, 4, 2> BigCfg;
// FP8 / MXFP8 256 x 256 tile: 8 waves of 128 x 64, BK 128, two 64 KB stages
// (one workgroup per CU), the byte layout of the bf16 Big tile
template <typename T> using BigCfg8 = Cfg<T, 256, 256, 128, 2, 4, 2>;
// FP8 weight gradients: 128 x 128, 4 waves of 64 x 64, BK 128, two stages;
// a workgroup runs up to kWgradRun column tiles of one row block
typedef Cfg<fp8_t, 128, 128, 128, 2, 2, 2> WgradCfg8;
typedef Cfg<mx8_t, 128, 128, 128, 2, 2, 2> WgradCfgMx8;
constexpr int kWgradRun = 8;
typedef Cfg<bf16_t, 128, 256, 32, 2, 2, 3> WgradCfg;

static int rows_tile_bound(int64_t A, int64_t G, int BM) {
  return int((A + G * (BM - 1)) / BM);
}


template <typename C, typename TC, bool AK, bool BKm, int MODE, int EPI>
static void run_gemm(GemmArgs g, int tiles, hipStream_t st) {
  if (tiles <= 0) return;
  if (MODE == G_KSPLIT) g.ksuper = super_wgrad(g.tiles_m * (g.tpw > 0 ? (g.tiles_n + g.tpw - 1) / g.tpw : g.tiles_n));
  else g.ksuper = super_rows(tiles / (g.G > 0 ? g.G : 1), C::BM);
  gemm_kernel<typename C::type, TC, AK, BKm, MODE, EPI, C::BM, C::BN, C::BK, C::WM, C::WN, C::NS>
      <<<padded_grid(tiles, g.ksuper), C::WM * C::WN * 64, 0, st>>>(g);
}

// Tile choice for the row-grouped GEMMs. The big tile halves operand traffic
// per flop but pads each expert's rows to a multiple of 256 and makes a
// quarter as many tiles: it is used when experts hold many rows (padding at
// most about half the rows) and the grid still has at least four rounds of
// tiles for the 256 CUs (measured: with two rounds of long-K tiles the
// ragged last round costs more than the big tile saves).
static int rows_tile_bound(int64_t A, int64_t G, int BM);
// `tile` (MOE_TILE_*: 0 auto, 1 small, 2 big) overrides the choice.
static bool big_rows(int tile, int64_t A, int64_t E, int64_t n_dim) {
  if (n_dim % 256 != 0 || tile == 1) return false;
  if (tile == 2) return true;
  return A >= 512 * E && int64_t(rows_tile_bound(A, E, 256)) * (n_dim / 256) >= 4 * 256;
}
// FP8 row-grouped GEMMs: the 256 x 256 tile only when forced (MOE_TILE_BIG)
// and the width allows.
static bool big8(int tile, int64_t n_dim) { return tile == 2 && n_dim % 256 == 0; }
// The 160-row tile (FP8, MXFP8 and bf16 row-grouped GEMMs) when experts
// average 120 to 320 rows: one row tile for experts of up to 160 rows, two
// up to 320, where the 128-row tile often needs one more for a few rows
// (measured on the FP8 DeepSeek-V3-style layer, 256 rows per expert:
// GEMM1 3.34 -> 3.13 ms, GEMM2 1.95 -> 1.79, dH 1.86 -> 1.73, dX 3.40 ->
// 3.22; a dense group of 8,192 rows lost 8 % on GEMM1 with it)
static bool mid8(int tile, int64_t A, int64_t E) { return tile == 0 && A >= 120 * E && A <= 320 * E; }
// Weight gradients tile the (M, N) = weight shape of every expert, whatever
// its rows: the big tile whenever the weight shape allows.
static bool big_wgrad(int tile, int64_t d, int64_t f) { return tile != 1 && d % 256 == 0 && f % 256 == 0; }

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

void launch_zero(void* dst, int64_t bytes, hipStream_t st) { zero_bytes(dst, bytes, st); }

// Workspace layout of the grouped FFN calls (byte offsets; see ffn_ws_bytes).
struct FfnWs {
  size_t h_bf16 = 0;   // fp8: H before quantisation [A, f] bf16 (fwd; bwd with recompute)
  size_t r_gu = 0;     // recompute 2, bwd: GU [A, 2f] act
  size_t r_h = 0;      // recompute: H [A, f] (act; fp8: E4M3 codes)
  size_t r_hs = 0;     // recompute, fp8: H scales [A, f/128]
  size_t d_gu = 0;     // bwd: dGU [A, 2f] act
  size_t d_out_q = 0;  // bwd fp8: dO codes [A, d] + scales [A, d/128]
  size_t d_out_s = 0;
  size_t d_gu_q = 0;   // bwd fp8: dGU codes [A, 2f] + scales [A, 2f/128]
  size_t d_gu_s = 0;
  // bwd fp8 and mxfp8: weight-gradient operands in token blocks: 128-row
  // block offsets [E+1], codes [A, C] and scales [NB, C] of dO, H, dGU and X
  size_t kblk = 0;
  size_t t_do = 0, t_do_s = 0, t_h = 0, t_h_s = 0, t_gu = 0, t_gu_s = 0, t_x = 0, t_x_s = 0;
  size_t total = 0;
};

static size_t al(size_t v) { return (v + 255) & ~size_t(255); }

static FfnWs ffn_ws(int64_t A, int64_t d, int64_t f, int64_t E, int act_bytes, int wt, bool bwd, int rc) {
  const bool fp8 = wt >= 2;
  FfnWs w;
  size_t o = 0;
  // H, when it is not kept between the calls, lives in the workspace: the
  // forward's GEMM2 operand, or the backward's rebuilt copy
  if (fp8 && (!bwd || rc)) { w.h_bf16 = o; o += al(size_t(A) * f * 2); }
  if (bwd && rc == 2) { w.r_gu = o; o += al(size_t(A) * 2 * f * act_bytes); }
  if (rc) {
    w.r_h = o; o += al(size_t(A) * f * (fp8 ? 1 : act_bytes));
    if (fp8) { w.r_hs = o; o += al(size_t(A) * (f / 128) * 4); }
  }
  if (bwd) {
    w.d_gu = o; o += al(size_t(A) * 2 * f * act_bytes);
    if (fp8) {
      w.d_out_q = o; o += al(size_t(A) * d);
      w.d_out_s = o; o += al(size_t(A) * (d / 128) * 4);
      w.d_gu_q = o; o += al(size_t(A) * 2 * f);
      w.d_gu_s = o; o += al(size_t(A) * (2 * f / 128) * 4);
      {
        // (MXFP8: the scale arrays hold one word of four E8M0 bytes per
        // 128-row block and column, the size of the FP8 fp32 scales)
        const size_t nb = size_t(token_blocks_bound(A, E));
        w.kblk = o; o += al(size_t(E + 1) * 4);
        w.t_do = o; o += al(size_t(A) * d);
        w.t_do_s = o; o += al(nb * d * 4);
        w.t_h = o; o += al(size_t(A) * f);
        w.t_h_s = o; o += al(nb * f * 4);
        w.t_gu = o; o += al(size_t(A) * 2 * f);
        w.t_gu_s = o; o += al(nb * 2 * f * 4);
        w.t_x = o; o += al(size_t(A) * d);
        w.t_x_s = o; o += al(nb * d * 4);
      }
    }
  }
  w.total = o;
  return w;
}

size_t ffn_ws_bytes(int64_t A, int64_t d, int64_t f, int64_t E, int act_bytes, int wt, bool bwd,
                    int recompute) {
  return ffn_ws(A, d, f, E, act_bytes, wt, bwd, recompute).total;
}

static char* at(void* base, size_t off) { return static_cast<char*>(base) + off; }

// GEMM1 (+ SwiGLU): GU = X W1^T (stored unless gu is null), H = silu(G) * U
template <typename C>
static void gemm1_fwd(const FfnLaunch& a, void* gu, void* h, hipStream_t st) {
  typedef typename C::type T;
  GemmArgs g1{};
  g1.A = a.x_perm; g1.lda = a.d;
  g1.B = a.w1; g1.ldb = a.d; g1.b_gstride = 2 * a.f * a.d;
  g1.offsets = a.offsets; g1.G = int(a.E);
  g1.N = int(2 * a.f); g1.K = int(a.d); g1.f = int(a.f);
  g1.aux0 = gu; g1.aux1 = h;
  g1.tiles_n = int(2 * a.f / C::BN);
  run_gemm<C, T, true, true, G_ROWS, EPI_SWIGLU>(g1, rows_tile_bound(a.A, a.E, C::BM) * g1.tiles_n, st);
}
// GEMM2: O = H W2^T
template <typename C>
static void gemm2_fwd(const FfnLaunch& a, const void* h, hipStream_t st) {
  typedef typename C::type T;
  GemmArgs g2{};
  g2.A = h; g2.lda = a.f;
  g2.B = a.w2; g2.ldb = a.f; g2.b_gstride = a.d * a.f;
  g2.C = a.out_perm; g2.ldc = a.d;
  g2.offsets = a.offsets; g2.G = int(a.E);
  g2.N = int(a.d); g2.K = int(a.f);
  g2.tiles_n = int(a.d / C::BN);
  run_gemm<C, T, true, true, G_ROWS, EPI_STORE>(g2, rows_tile_bound(a.A, a.E, C::BM) * g2.tiles_n, st);
}

// FP8 GEMM1 (+ SwiGLU) into h16 (bf16), then H -> E4M3 per 1 x 128 block
// (the second GEMM's A operand; the weight gradient requantises it in token
// blocks)
template <typename C>
static void gemm1_fwd_fp8(const FfnLaunch& a, void* gu, bf16_t* h16, uint8_t* hq, float* hs,
                          hipStream_t st) {
  GemmArgs g1{};
  g1.A = a.x_perm; g1.lda = a.d;
  g1.a_scale = a.x_scale; g1.a_scale_ld = int(a.d / 128);
  g1.B = a.w1; g1.ldb = a.d; g1.b_gstride = 2 * a.f * a.d;
  g1.b_scale = a.w1_scale; g1.b_scale_gstride = (2 * a.f / 128) * (a.d / 128); g1.b_scale_ld = int(a.d / 128);
  g1.offsets = a.offsets; g1.G = int(a.E);
  g1.N = int(2 * a.f); g1.K = int(a.d); g1.f = int(a.f);
  g1.aux0 = gu; g1.aux1 = h16;
  g1.tiles_n = int(2 * a.f / C::BN);
  run_gemm<C, bf16_t, true, true, G_ROWS, EPI_SWIGLU>(g1, rows_tile_bound(a.A, a.E, C::BM) * g1.tiles_n, st);
  launch_quant_rows(h16, true, a.A, a.f, hq, hs, st);
}

template <typename C>
static void gemm2_fwd_fp8(const FfnLaunch& a, const uint8_t* hq, const float* hs, hipStream_t st) {
  GemmArgs g2{};
  g2.A = hq; g2.lda = a.f;
  g2.a_scale = hs; g2.a_scale_ld = int(a.f / 128);
  g2.B = a.w2; g2.ldb = a.f; g2.b_gstride = a.d * a.f;
  g2.b_scale = a.w2_scale; g2.b_scale_gstride = (a.d / 128) * (a.f / 128); g2.b_scale_ld = int(a.f / 128);
  g2.C = a.out_perm; g2.ldc = a.d;
  g2.offsets = a.offsets; g2.G = int(a.E);
  g2.N = int(a.d); g2.K = int(a.f);
  g2.tiles_n = int(a.d / C::BN);
  run_gemm<C, bf16_t, true, true, G_ROWS, EPI_STORE>(g2, rows_tile_bound(a.A, a.E, C::BM) * g2.tiles_n, st);
}

// MXFP8 GEMMs: scale words of 4 E8M0 bytes per A row (a_scale_ld = K / 128
// words); B scales in bytes: rows of K / 32 for K-major weights (the forward's
// row-quantised W1, W2), rows of N per 32-deep K block for K-strided weights
// (the data gradients' column-quantised W2, W1).
template <typename C>
static void gemm1_fwd_mx(const FfnLaunch& a, void* gu, bf16_t* h16, uint8_t* hq, uint8_t* hs, hipStream_t st) {
  GemmArgs g1{};
  g1.A = a.x_perm; g1.lda = a.d;
  g1.a_scale = a.x_scale; g1.a_scale_ld = int(a.d / 128);
  g1.B = a.w1; g1.ldb = a.d; g1.b_gstride = 2 * a.f * a.d;
  g1.b_scale = a.w1_scale; g1.b_scale_gstride = 2 * a.f * (a.d / 32); g1.b_scale_ld = int(a.d / 32);
  g1.offsets = a.offsets; g1.G = int(a.E);
  g1.N = int(2 * a.f); g1.K = int(a.d); g1.f = int(a.f);
  g1.aux0 = gu; g1.aux1 = h16;
  g1.tiles_n = int(2 * a.f / C::BN);
  run_gemm<C, bf16_t, true, true, G_ROWS, EPI_SWIGLU>(g1, rows_tile_bound(a.A, a.E, C::BM) * g1.tiles_n, st);
  launch_quant_mx_rows(h16, true, a.A, a.f, hq, hs, st);
}

template <typename C>
static void gemm2_fwd_mx(const FfnLaunch& a, const uint8_t* hq, const uint8_t* hs, hipStream_t st) {
  GemmArgs g2{};
  g2.A = hq; g2.lda = a.f;
  g2.a_scale = reinterpret_cast<const float*>(hs); g2.a_scale_ld = int(a.f / 128);
  g2.B = a.w2; g2.ldb = a.f; g2.b_gstride = a.d * a.f;
  g2.b_scale = a.w2_scale; g2.b_scale_gstride = a.d * (a.f / 32); g2.b_scale_ld = int(a.f / 32);
  g2.C = a.out_perm; g2.ldc = a.d;
  g2.offsets = a.offsets; g2.G = int(a.E);
  g2.N = int(a.d); g2.K = int(a.f);
  g2.tiles_n = int(a.d / C::BN);
  run_gemm<C, bf16_t, true, true, G_ROWS, EPI_STORE>(g2, rows_tile_bound(a.A, a.E, C::BM) * g2.tiles_n, st);
}

// The first half of the forward: GU (into gu unless null) and H (+ scales).
static void ffn_fwd_gu_h(const FfnLaunch& a, void* gu, void* h, float* hs, bf16_t* h16, hipStream_t st) {
  if (a.wt == 3) {
    if (mid8(a.tile, a.A, a.E))
      gemm1_fwd_mx<MidCfg8<mx8_t>>(a, gu, h16, static_cast<uint8_t*>(h), reinterpret_cast<uint8_t*>(hs), st);
    else
      gemm1_fwd_mx<SmallCfg<mx8_t>>(a, gu, h16, static_cast<uint8_t*>(h), reinterpret_cast<uint8_t*>(hs), st);
  } else if (a.wt == 2) {
    if (big8(a.tile, 2 * a.f)) gemm1_fwd_fp8<BigCfg8<fp8_t>>(a, gu, h16, static_cast<uint8_t*>(h), hs, st);
    else if (mid8(a.tile, a.A, a.E)) gemm1_fwd_fp8<MidCfg8<fp8_t>>(a, gu, h16, static_cast<uint8_t*>(h), hs, st);
    else gemm1_fwd_fp8<SmallCfg<fp8_t>>(a, gu, h16, static_cast<uint8_t*>(h), hs, st);
  } else if (a.wt == 1) {
    if (big_rows(a.tile, a.A, a.E, 2 * a.f)) gemm1_fwd<BigCfg>(a, gu, h, st);
    else if (mid8(a.tile, a.A, a.E)) gemm1_fwd<MidCfg16>(a, gu, h, st);
    else gemm1_fwd<SmallCfg<bf16_t>>(a, gu, h, st);
  } else {
    gemm1_fwd<SmallCfg<float>>(a, gu, h, st);
  }
}

// Weight gradients over the ragged rows of every expert (K split by group).
template <typename C, typename TW>
static void wgrad_t(const void* d_out, const void* act_h, const void* d_gu, const void* x, void* dw1,
                    void* dw2, const int32_t* offsets, int64_t d, int64_t f, int64_t E, hipStream_t st) {
  constexpr bool persist = persistent_wgrad<typename C::type, TW, G_KSPLIT, EPI_STORE, C::NS>();
  // persistent instances: runs of column tiles while the grid keeps at least
  // 8 workgroups per CU
  auto grid = [&](GemmArgs& gg) {
    if (!persist) return int(E) * gg.tiles_m * gg.tiles_n;
    gg.tpw = int(std::max<int64_t>(1, std::min<int64_t>(kWgradRun, E * gg.tiles_m * gg.tiles_n / 2048)));
    return int(E) * gg.tiles_m * ((gg.tiles_n + gg.tpw - 1) / gg.tpw);
  };
  // dW2 = dO^T H   [d, f]
  GemmArgs g3{};
  g3.A = d_out; g3.lda = d;
  g3.B = act_h; g3.ldb = f;
  g3.C = dw2; g3.ldc = f; g3.c_gstride = d * f;
  g3.offsets = offsets; g3.G = int(E);
  g3.M = int(d); g3.N = int(f);
  g3.tiles_m = int(d / C::BM); g3.tiles_n = int(f / C::BN);
  const int n3 = grid(g3);  // sets g3.tpw before the copy run_gemm takes
  run_gemm<C, TW, false, false, G_KSPLIT, EPI_STORE>(g3, n3, st);
  // dW1 = dGU^T X   [2f, d]
  GemmArgs g4{};
  g4.A = d_gu; g4.lda = 2 * f;
  g4.B = x; g4.ldb = d;
  g4.C = dw1; g4.ldc = d; g4.c_gstride = 2 * f * d;
  g4.offsets = offsets; g4.G = int(E);
  g4.M = int(2 * f); g4.N = int(d);
  g4.tiles_m = int(2 * f / C::BM); g4.tiles_n = int(d / C::BN);
  const int n4 = grid(g4);
  run_gemm<C, TW, false, false, G_KSPLIT, EPI_STORE>(g4, n4, st);
}

// 8-bit weight gradients: dW2 = dO^T H and dW1 = dGU^T X with every operand
// in token blocks (codes [A, C], scales [NB, C] per 128-row block and
// column: FP8 fp32 scales of 128-row x 1 blocks, or MXFP8 words of four
// 32-row E8M0 bytes; kblk the first block of each expert); bf16 results.
template <bool MXF>
static void wgrad_8bit(const fp8_t* dq, const void* ds, const fp8_t* hq, const void* hs, const fp8_t* gq,
                       const void* gs, const fp8_t* xq, const void* xs, const int32_t* kblk, void* dw1, void* dw2,
                       const int32_t* offsets, int64_t d, int64_t f, int64_t E, hipStream_t st) {
  typedef std::conditional_t<MXF, WgradCfgMx8, WgradCfg8> C;
  auto sc = [](const void* p) { return static_cast<const float*>(p); };
  auto run = [&](GemmArgs& gg) {
    // runs of column tiles while the grid keeps at least 8 workgroups per CU
    const int64_t tiles = E * gg.tiles_m * gg.tiles_n;
    gg.tpw = int(std::max<int64_t>(1, std::min<int64_t>(kWgradRun, tiles / 2048)));
    run_gemm<C, bf16_t, false, false, G_KSPLIT, EPI_STORE>(
        gg, int(E) * gg.tiles_m * ((gg.tiles_n + gg.tpw - 1) / gg.tpw), st);
  };
  GemmArgs g3{};
  g3.A = dq; g3.lda = d; g3.a_scale = sc(ds); g3.a_scale_ld = int(d);
  g3.B = hq; g3.ldb = f; g3.b_scale = sc(hs); g3.b_scale_ld = int(f);
  g3.kblk = kblk;
  g3.C = dw2; g3.ldc = f; g3.c_gstride = d * f;
  g3.offsets = offsets; g3.G = int(E);
  g3.M = int(d); g3.N = int(f);
  g3.tiles_m = int(d / C::BM); g3.tiles_n = int(f / C::BN);
  run(g3);
  GemmArgs g4{};
  g4.A = gq; g4.lda = 2 * f; g4.a_scale = sc(gs); g4.a_scale_ld = int(2 * f);
  g4.B = xq; g4.ldb = d; g4.b_scale = sc(xs); g4.b_scale_ld = int(d);
  g4.kblk = kblk;
  g4.C = dw1; g4.ldc = d; g4.c_gstride = 2 * f * d;
  g4.offsets = offsets; g4.G = int(E);
  g4.M = int(2 * f); g4.N = int(d);
  g4.tiles_m = int(2 * f / C::BM); g4.tiles_n = int(d / C::BN);
  run(g4);
}

// bf16 weight gradients: experts of a few hundred rows (a few K steps per
// tile, so each tile is mostly its result stores) take the persistent
// column-tile runs of the 128 x 128 tile, whose next tile's loads overlap a
// tile's stores; longer experts the 128 x 256 three-stage tile.
static bool persist_wgrad_bf16(int tile, int64_t A, int64_t E) { return tile != 2 && A <= 256 * E; }

template <typename TC16>
static void wgrad_any(int tile, const void* d_out, const void* act_h, const void* d_gu, const void* x, void* dw1,
                      void* dw2, const int32_t* offsets, int64_t A, int64_t d, int64_t f, int64_t E,
                      hipStream_t st) {
  if (!persist_wgrad_bf16(tile, A, E) && big_wgrad(tile, d, f))
    wgrad_t<WgradCfg, TC16>(d_out, act_h, d_gu, x, dw1, dw2, offsets, d, f, E, st);
  else
    wgrad_t<SmallCfg<bf16_t>, TC16>(d_out, act_h, d_gu, x, dw1, dw2, offsets, d, f, E, st);
}

// dH = dO W2, fused SwiGLU backward -> dGU (and H rebuilt into h_out unless null)
template <typename C>
static void dh_bwd(const FfnBwdLaunch& a, void* d_gu, void* h_out, hipStream_t st) {
  typedef typename C::type T;
  GemmArgs g1{};
  g1.A = a.d_out; g1.lda = a.d;
  g1.B = a.w2; g1.ldb = a.f; g1.b_gstride = a.d * a.f;
  g1.C = d_gu; g1.ldc = 2 * a.f;
  g1.offsets = a.offsets; g1.G = int(a.E);
  g1.N = int(a.f); g1.K = int(a.d); g1.f = int(a.f);
  g1.aux0 = const_cast<void*>(a.act_gu); g1.aux1 = h_out;
  g1.tiles_n = int(a.f / C::BN);
  run_gemm<C, T, true, false, G_ROWS, EPI_DSWIGLU>(g1, rows_tile_bound(a.A, a.E, C::BM) * g1.tiles_n, st);
}
// dX = dGU W1
template <typename C>
static void dx_bwd(const FfnBwdLaunch& a, const void* d_gu, hipStream_t st) {
  typedef typename C::type T;
  GemmArgs g2{};
  g2.A = d_gu; g2.lda = 2 * a.f;
  g2.B = a.w1; g2.ldb = a.d; g2.b_gstride = 2 * a.f * a.d;
  g2.C = a.dx_perm; g2.ldc = a.d;
  g2.offsets = a.offsets; g2.G = int(a.E);
  g2.N = int(a.d); g2.K = int(2 * a.f);
  g2.tiles_n = int(a.d / C::BN);
  run_gemm<C, T, true, false, G_ROWS, EPI_STORE>(g2, rows_tile_bound(a.A, a.E, C::BM) * g2.tiles_n, st);
}

// a.act_h is the saved H, or, with h_out set (activation recompute), the
// buffer the dH GEMM's epilogue rebuilds H into from the saved GU.
template <typename T>
static void ffn_bwd_t(const FfnBwdLaunch& a, void* h_out, hipStream_t st) {
  const FfnWs w = ffn_ws(a.A, a.d, a.f, a.E, int(sizeof(T)), a.wt, true, a.recompute);
  void* d_gu = at(a.ws, w.d_gu);
  if constexpr (sizeof(T) == 2) {
    if (big_rows(a.tile, a.A, a.E, a.f)) dh_bwd<BigCfg>(a, d_gu, h_out, st);
    else if (mid8(a.tile, a.A, a.E)) dh_bwd<MidCfg16>(a, d_gu, h_out, st);
    else dh_bwd<SmallCfg<bf16_t>>(a, d_gu, h_out, st);
    if (big_rows(a.tile, a.A, a.E, a.d)) dx_bwd<BigCfg>(a, d_gu, st);
    else if (mid8(a.tile, a.A, a.E)) dx_bwd<MidCfg16>(a, d_gu, st);
    else dx_bwd<SmallCfg<bf16_t>>(a, d_gu, st);
    wgrad_any<bf16_t>(a.tile, a.d_out, a.act_h, d_gu, a.x_perm, a.dw1, a.dw2, a.offsets, a.A, a.d, a.f, a.E, st);
  } else {
    dh_bwd<SmallCfg<float>>(a, d_gu, h_out, st);
    dx_bwd<SmallCfg<float>>(a, d_gu, st);
    wgrad_t<SmallCfg<float>, float>(a.d_out, a.act_h, d_gu, a.x_perm, a.dw1, a.dw2, a.offsets, a.d, a.f,
                                     a.E, st);
  }
}

// 8-bit backward: the data-gradient GEMMs run with their gradient operand
// quantised in row blocks along the contraction dim (FP8: 1 x 128 with fp32
// scales and the forward's 128 x 128 weight blocks; MXFP8 (MXF): 1 x 32 E8M0
// blocks and the column-quantised weight copies, 32 x 1 blocks along these
// products' contraction dims, that the caller passes as w1, w2). The weight
// gradients take all four operands in token blocks inside each expert's rows
// (FP8: 128-row x 1 with fp32 scales; MXFP8: 32-row x 1 E8M0 blocks, four to
// a scale word), X and H requantised from their forward codes. With h16 set
// (activation recompute) the dH epilogue rebuilds H in bf16 from the saved
// GU and it is quantised as in the forward into a.act_h / a.h_scale.
// FP8 / MXFP8 data gradients: dH = Q(dO) W2 (+ SwiGLU backward from the
// saved bf16 GU; H rebuilt into h16 unless null) and dX = Q(dGU) W1, on
// tile configuration C.
template <bool MXF, typename C>
static void dh_fp8(const FfnBwdLaunch& a, const uint8_t* dq, const float* ds, bf16_t* d_gu, bf16_t* h16,
                   hipStream_t st) {
  GemmArgs g1{};
  g1.A = dq; g1.lda = a.d;
  g1.a_scale = ds; g1.a_scale_ld = int(a.d / 128);
  g1.B = a.w2; g1.ldb = a.f; g1.b_gstride = a.d * a.f;
  g1.b_scale = a.w2_scale;
  if constexpr (MXF) { g1.b_scale_gstride = (a.d / 32) * a.f; g1.b_scale_ld = int(a.f); }
  else { g1.b_scale_gstride = (a.d / 128) * (a.f / 128); g1.b_scale_ld = int(a.f / 128); }
  g1.C = d_gu; g1.ldc = 2 * a.f;
  g1.offsets = a.offsets; g1.G = int(a.E);
  g1.N = int(a.f); g1.K = int(a.d); g1.f = int(a.f);
  g1.aux0 = const_cast<void*>(a.act_gu); g1.aux1 = h16;
  g1.tiles_n = int(a.f / C::BN);
  run_gemm<C, bf16_t, true, false, G_ROWS, EPI_DSWIGLU>(g1, rows_tile_bound(a.A, a.E, C::BM) * g1.tiles_n, st);
}
template <bool MXF, typename C>
static void dx_fp8(const FfnBwdLaunch& a, const uint8_t* gq, const float* gs, hipStream_t st) {
  GemmArgs g2{};
  g2.A = gq; g2.lda = 2 * a.f;
  g2.a_scale = gs; g2.a_scale_ld = int(2 * a.f / 128);
  g2.B = a.w1; g2.ldb = a.d; g2.b_gstride = 2 * a.f * a.d;
  g2.b_scale = a.w1_scale;
  if constexpr (MXF) { g2.b_scale_gstride = (2 * a.f / 32) * a.d; g2.b_scale_ld = int(a.d); }
  else { g2.b_scale_gstride = (2 * a.f / 128) * (a.d / 128); g2.b_scale_ld = int(a.d / 128); }
  g2.C = a.dx_perm; g2.ldc = a.d;
  g2.offsets = a.offsets; g2.G = int(a.E);
  g2.N = int(a.d); g2.K = int(2 * a.f);
  g2.tiles_n = int(a.d / C::BN);
  run_gemm<C, bf16_t, true, false, G_ROWS, EPI_STORE>(g2, rows_tile_bound(a.A, a.E, C::BM) * g2.tiles_n, st);
}

template <bool MXF>
static void ffn_bwd_fp8(const FfnBwdLaunch& a, bf16_t* h16, hipStream_t st) {
  typedef std::conditional_t<MXF, mx8_t, fp8_t> T8;
  auto quant = [&](const void* src, int64_t rows, int64_t cols, uint8_t* q, float* sc) {
    if constexpr (MXF) launch_quant_mx_rows(src, true, rows, cols, q, reinterpret_cast<uint8_t*>(sc), st);
    else launch_quant_rows(src, true, rows, cols, q, sc, st);
  };
  const FfnWs w = ffn_ws(a.A, a.d, a.f, a.E, 2, a.wt, true, a.recompute);
  bf16_t* d_gu = reinterpret_cast<bf16_t*>(at(a.ws, w.d_gu));
  uint8_t* dq = reinterpret_cast<uint8_t*>(at(a.ws, w.d_out_q));
  float* ds = reinterpret_cast<float*>(at(a.ws, w.d_out_s));
  uint8_t* gq = reinterpret_cast<uint8_t*>(at(a.ws, w.d_gu_q));
  float* gs = reinterpret_cast<float*>(at(a.ws, w.d_gu_s));
  int32_t* kblk = reinterpret_cast<int32_t*>(at(a.ws, w.kblk));
  auto tq = [&](size_t o) { return reinterpret_cast<fp8_t*>(at(a.ws, o)); };
  auto ts = [&](size_t o) { return reinterpret_cast<float*>(at(a.ws, o)); };
  auto tw = [&](size_t o) { return reinterpret_cast<uint32_t*>(at(a.ws, o)); };
  if constexpr (MXF) {
    // dO read once: its 1 x 32 row blocks (dH) and 32-row blocks (dW2)
    kblock_offsets_kernel<<<1, 1024, 0, st>>>(a.offsets, kblk, int(a.E));
    quant_tokens_mx(a.d_out, nullptr, a.offsets, kblk, a.E, a.A, a.d, tq(w.t_do), tw(w.t_do_s), st, dq,
                    reinterpret_cast<uint8_t*>(ds));
  } else {
    // dO read once: its 1 x 128 row blocks (dH) and 128-row blocks (dW2)
    kblock_offsets_kernel<<<1, 1024, 0, st>>>(a.offsets, kblk, int(a.E));
    quant_tokens(a.d_out, nullptr, a.offsets, kblk, a.E, a.A, a.d, tq(w.t_do), ts(w.t_do_s), st, dq, ds);
  }
  // dH = Q(dO) W2 (+ SwiGLU backward from the saved bf16 GU)
  // (the MXFP8 instance keeps the 128 x 128 tile: its per-lane scale words
  // do not fit the 256 x 256 tile's registers)
  if constexpr (!MXF) {
    if (big8(a.tile, a.f)) dh_fp8<MXF, BigCfg8<T8>>(a, dq, ds, d_gu, h16, st);
    else if (mid8(a.tile, a.A, a.E)) dh_fp8<MXF, MidCfg8<T8>>(a, dq, ds, d_gu, h16, st);
    else dh_fp8<MXF, SmallCfg<T8>>(a, dq, ds, d_gu, h16, st);
  } else {
    if (mid8(a.tile, a.A, a.E)) dh_fp8<MXF, MidCfg8<T8>>(a, dq, ds, d_gu, h16, st);
    else dh_fp8<MXF, SmallCfg<T8>>(a, dq, ds, d_gu, h16, st);
  }
  if (h16) quant(h16, a.A, a.f, static_cast<uint8_t*>(const_cast<void*>(a.act_h)), const_cast<float*>(a.h_scale));
  // dX = Q(dGU) W1
  if constexpr (MXF) {
    quant_tokens_mx(d_gu, nullptr, a.offsets, kblk, a.E, a.A, 2 * a.f, tq(w.t_gu), tw(w.t_gu_s), st, gq,
                    reinterpret_cast<uint8_t*>(gs));
  } else {
    quant_tokens(d_gu, nullptr, a.offsets, kblk, a.E, a.A, 2 * a.f, tq(w.t_gu), ts(w.t_gu_s), st, gq, gs);
  }
  if constexpr (!MXF) {
    if (big8(a.tile, a.d)) dx_fp8<MXF, BigCfg8<T8>>(a, gq, gs, st);
    else if (mid8(a.tile, a.A, a.E)) dx_fp8<MXF, MidCfg8<T8>>(a, gq, gs, st);
    else dx_fp8<MXF, SmallCfg<T8>>(a, gq, gs, st);
  } else {
    if (mid8(a.tile, a.A, a.E)) dx_fp8<MXF, MidCfg8<T8>>(a, gq, gs, st);
    else dx_fp8<MXF, SmallCfg<T8>>(a, gq, gs, st);
  }
  if constexpr (MXF) {
    // weight gradients in MXFP8: the four operands in 32-row x 1 blocks,
    // H and X from their forward codes
    const uint8_t* hs8 = reinterpret_cast<const uint8_t*>(a.h_scale);
    const uint8_t* xs8 = reinterpret_cast<const uint8_t*>(a.x_scale);
    quant_tokens_mx(a.act_h, hs8, a.offsets, kblk, a.E, a.A, a.f, tq(w.t_h), tw(w.t_h_s), st);
    quant_tokens_mx(a.x_perm, xs8, a.offsets, kblk, a.E, a.A, a.d, tq(w.t_x), tw(w.t_x_s), st);
  } else {
    // weight gradients in FP8: the four operands in 128-row x 1 blocks (dO
    // and dGU were quantised so with their row blocks)
    quant_tokens(a.act_h, a.h_scale, a.offsets, kblk, a.E, a.A, a.f, tq(w.t_h), ts(w.t_h_s), st);
    quant_tokens(a.x_perm, a.x_scale, a.offsets, kblk, a.E, a.A, a.d, tq(w.t_x), ts(w.t_x_s), st);
  }
  wgrad_8bit<MXF>(tq(w.t_do), at(a.ws, w.t_do_s), tq(w.t_h), at(a.ws, w.t_h_s), tq(w.t_gu), at(a.ws, w.t_gu_s),
                  tq(w.t_x), at(a.ws, w.t_x_s), kblk, a.dw1, a.dw2, a.offsets, a.d, a.f, a.E, st);
}

void launch_grouped_ffn(const FfnLaunch& a, hipStream_t st) {
  if (a.identity) {
    copy_bytes(a.x_perm, a.out_perm, a.A * a.d * (a.act == 1 ? 2 : 4), st);
    return;
  }
  const FfnWs w = ffn_ws(a.A, a.d, a.f, a.E, a.act == 1 ? 2 : 4, a.wt, false, a.recompute);
  // what the backward will not find saved goes to the workspace (H) or is
  // not stored at all (GU)
  void* gu = a.recompute == 2 ? nullptr : a.act_gu;
  void* h = a.recompute ? at(a.ws, w.r_h) : a.act_h;
  float* hs = a.recompute ? reinterpret_cast<float*>(at(a.ws, w.r_hs)) : a.h_scale;
  bf16_t* h16 = reinterpret_cast<bf16_t*>(at(a.ws, w.h_bf16));
  ffn_fwd_gu_h(a, gu, h, hs, h16, st);
  if (a.wt == 3) {
    if (mid8(a.tile, a.A, a.E))
      gemm2_fwd_mx<MidCfg8<mx8_t>>(a, static_cast<const uint8_t*>(h), reinterpret_cast<const uint8_t*>(hs), st);
    else
      gemm2_fwd_mx<SmallCfg<mx8_t>>(a, static_cast<const uint8_t*>(h), reinterpret_cast<const uint8_t*>(hs), st);
  } else if (a.wt == 2) {
    if (big8(a.tile, a.d)) gemm2_fwd_fp8<BigCfg8<fp8_t>>(a, static_cast<const uint8_t*>(h), hs, st);
    else if (mid8(a.tile, a.A, a.E)) gemm2_fwd_fp8<MidCfg8<fp8_t>>(a, static_cast<const uint8_t*>(h), hs, st);
    else gemm2_fwd_fp8<SmallCfg<fp8_t>>(a, static_cast<const uint8_t*>(h), hs, st);
  } else if (a.wt == 1) {
    if (big_rows(a.tile, a.A, a.E, a.d)) gemm2_fwd<BigCfg>(a, h, st);
    else if (mid8(a.tile, a.A, a.E)) gemm2_fwd<MidCfg16>(a, h, st);
    else gemm2_fwd<SmallCfg<bf16_t>>(a, h, st);
  } else {
    gemm2_fwd<SmallCfg<float>>(a, h, st);
  }
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
  const bool fp8 = a.wt >= 2;
  const FfnWs w = ffn_ws(a.A, a.d, a.f, a.E, es, a.wt, true, a.recompute);
  FfnBwdLaunch b = a;
  void* h_out = nullptr;  // activation recompute: H rebuilt by the dH epilogue
  if (a.recompute) {
    b.act_h = at(a.ws, w.r_h);
    b.h_scale = reinterpret_cast<const float*>(at(a.ws, w.r_hs));
    bf16_t* h16 = reinterpret_cast<bf16_t*>(at(a.ws, w.h_bf16));
    if (a.recompute == 2) {
      // rerun the forward's first GEMM: GU and H exactly as the forward made them
      FfnLaunch f{};
      f.x_perm = a.x_perm; f.x_scale = a.x_scale; f.offsets = a.offsets;
      f.w1 = a.w1; f.w1_scale = a.w1_scale;
      f.A = a.A; f.d = a.d; f.f = a.f; f.E = a.E; f.act = a.act; f.wt = a.wt; f.tile = a.tile;
      b.act_gu = at(a.ws, w.r_gu);
      ffn_fwd_gu_h(f, const_cast<void*>(b.act_gu), const_cast<void*>(b.act_h),
                   const_cast<float*>(b.h_scale), h16, st);
    } else {
      h_out = fp8 ? static_cast<void*>(h16) : const_cast<void*>(b.act_h);
    }
  }
  if (a.wt == 3) ffn_bwd_fp8<true>(b, static_cast<bf16_t*>(h_out), st);
  else if (fp8) ffn_bwd_fp8<false>(b, static_cast<bf16_t*>(h_out), st);
  else if (a.wt == 1) ffn_bwd_t<bf16_t>(b, h_out, st);
  else ffn_bwd_t<float>(b, h_out, st);
}

}  // namespace moe

// Router forward and backward kernels (gfx950).
//
// Router scoring, top-k selection and gates: a router chooses a few experts
// per token (Megatron Core MoE summary, "O essencial" and technical summary
// section 1); routing is fused with the permutation bookkeeping to cut
// launches (same page, section 2.4, kernel fusion).
//
// The logits use a fixed fp32 order so that selection is reproducible bit for
// bit: every output is its own fused multiply-add recurrence over the hidden
// index in ascending order. Work is split over outputs only (no split of the
// hidden dimension, no cross-lane sum), staged through LDS in chunks.
//
// This file is compiled with -ffp-contract=off.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

// ---------------------------------------------------------------------------
// Router backward products on the fp32 matrix cores (v_mfma_f32_16x16x4f32):
//   C(m, n) (op)= sum_k A(m, k) B(k, n) over the block's contraction range
//   A fp32:  A_MK: A(m,k) = A[m*lda + k], else A[k*lda + m]
//   B (f32 or bf16, widened exactly): B(k,n) = B[k*ldb + n]
//   EPI store: fp32 C[z*c_zstride + m*ldc + n]; EPI add: C (act dtype) += v,
//   one rounding.
// The backward has no bit-exactness requirement (unlike the logits); the
// summation order is fixed by the tiling, so results are deterministic.
// Tile 64 x 128 (4 waves of 32 x 64), contraction chunks of 32 staged in
// LDS; the next chunk is loaded into registers while the current one is
// multiplied.
// ---------------------------------------------------------------------------
enum { VEPI_STORE = 0, VEPI_ADD_ACT = 1 };

struct VArgs {
  const void* A;
  int64_t lda;
  const void* B;
  int64_t ldb;
  void* C;
  int64_t ldc;
  int M, N, K;
  int kchunk;         // contraction range of blockIdx.z: [z*kchunk, (z+1)*kchunk)
  int64_t c_zstride;  // elements between the partial outputs of consecutive z
};

template <typename T>
__device__ __forceinline__ float ld_elem(const void* p, int64_t i) {
  return Elem<T>::load(reinterpret_cast<const T*>(p) + i);
}

constexpr int kRgBM = 64, kRgBN = 128, kRgBK = 32;

// Epilogue of the router-backward products (acc: a lane holds rows
// 4 (l / 16) + r, column l % 16 of each 16 x 16 block of its 32 x 64 part).
template <typename TC, int EPI>
__device__ __forceinline__ void rgemm_epilogue(const VArgs& a, const f32x4_t (&acc)[2][4], float* Cs, int m0, int n0,
                                               int wm, int wn, int wave, int lane) {
  if constexpr (EPI == VEPI_STORE) {
    // fp32 partial sums: 16 lanes store 64 contiguous bytes
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int gn = n0 + wn * 64 + j * 16 + lane % 16;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int gm = m0 + wm * 32 + i * 16 + 4 * (lane / 16) + r;
          if (gm < a.M && gn < a.N)
            reinterpret_cast<float*>(a.C)[blockIdx.z * a.c_zstride + int64_t(gm) * a.ldc + gn] = acc[i][j][r];
        }
      }
    return;
  }
  // Add into the activation gradient through LDS: each wave stages 16 rows x
  // 64 columns at a time and reads them back as 8 consecutive columns per
  // lane, for 16-byte read-modify-write accesses.
  constexpr int EP = 64 + 4;
  float* stg = Cs + wave * 16 * EP;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) stg[(4 * (lane / 16) + r) * EP + j * 16 + lane % 16] = acc[i][j][r];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int u = lane + 64 * h, rr = u / 8, c8 = (u % 8) * 8;
      const int gm = m0 + wm * 32 + i * 16 + rr, gn = n0 + wn * 64 + c8;
      if (gm >= a.M) continue;
      float v[8];
      const float4 lo = *reinterpret_cast<const float4*>(&stg[rr * EP + c8]);
      const float4 hi = *reinterpret_cast<const float4*>(&stg[rr * EP + c8 + 4]);
      v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w; v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
      TC* c = reinterpret_cast<TC*>(a.C) + int64_t(gm) * a.ldc + gn;
      if (gn + 8 <= a.N) {
        constexpr int VC = 16 / int(sizeof(TC));
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; e += VC) Vec16<TC>::load(c + e, o + e);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = o[e] + v[e];
#pragma unroll
        for (int e = 0; e < 8; e += VC) Vec16<TC>::store(c + e, o + e);
      } else {
        for (int e = 0; e < 8; ++e)
          if (gn + e < a.N) Elem<TC>::store(c + e, Elem<TC>::load(c + e) + v[e]);
      }
    }
  }
}

template <typename TB, bool A_MK, typename TC, int EPI>
__global__ __launch_bounds__(256) void rgemm_kernel(VArgs a) {
  constexpr int BM = kRgBM, BN = kRgBN, BK = kRgBK;
  constexpr int PA = BM + 4, PB = BN + 4;   // LDS pitches (floats; rows stay 16-byte aligned)
  constexpr int VB = 16 / int(sizeof(TB));  // B elements per 16-byte load
  constexpr int NA = BM * BK / 4 / 256;     // 4-float groups of A per thread
  constexpr int NB = BN * BK / VB / 256;    // 16-byte groups of B per thread
  __shared__ __attribute__((aligned(16))) float As[BK * PA];  // [k][m]
  __shared__ __attribute__((aligned(16))) float Bs[BK * PB];  // [k][n]
  // epilogue staging of the read-modify-write (add) variant
  __shared__ __attribute__((aligned(16))) float Cs[EPI == VEPI_ADD_ACT ? 4 * 16 * (64 + 4) : 4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int kb = blockIdx.z * a.kchunk;
  const int ke = min(a.K, kb + a.kchunk);
  const float* A = reinterpret_cast<const float*>(a.A);
  // 16-byte loads along A's contiguous index (A_MK: chunk starts stay 4-aligned)
  const bool a_vec = (a.lda & 3) == 0 && (!A_MK || (a.kchunk & 3) == 0);
  // A group i: 4 values along A's contiguous index (k when A_MK, else m)
  auto a_pos = [&](int i, int& m, int& kk) {
    const int q = (tid + 256 * i) * 4;
    if (A_MK) { m = q / BK; kk = q % BK; } else { kk = q / BM; m = q % BM; }
  };
  float ra[NA][4], rb[NB][VB];
  auto gload = [&](int k0) {
    // a chunk inside M, N and the K range (uniform over the workgroup):
    // every load unconditional, so they all go out together; under the
    // per-load bounds branches below each one was waited for alone
    if (a_vec && m0 + BM <= a.M && n0 + BN <= a.N && k0 + BK <= ke) {
#pragma unroll
      for (int i = 0; i < NA; ++i) {
        int m, kk;
        a_pos(i, m, kk);
        const float4 v = *reinterpret_cast<const float4*>(A_MK ? A + int64_t(m0 + m) * a.lda + k0 + kk
                                                                : A + int64_t(k0 + kk) * a.lda + m0 + m);
        ra[i][0] = v.x; ra[i][1] = v.y; ra[i][2] = v.z; ra[i][3] = v.w;
      }
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int q = (tid + 256 * i) * VB;
        Vec16<TB>::load(reinterpret_cast<const TB*>(a.B) + int64_t(k0 + q / BN) * a.ldb + n0 + q % BN, rb[i]);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      int m, kk;
      a_pos(i, m, kk);
      const int gm = m0 + m, gk = k0 + kk;
      const bool full = A_MK ? (gm < a.M && gk + 4 <= ke) : (gk < ke && gm + 4 <= a.M);
      if (full && a_vec) {
        const float4 v = *reinterpret_cast<const float4*>(A_MK ? A + int64_t(gm) * a.lda + gk
                                                                : A + int64_t(gk) * a.lda + gm);
        ra[i][0] = v.x; ra[i][1] = v.y; ra[i][2] = v.z; ra[i][3] = v.w;
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int mm = A_MK ? gm : gm + j, kq = A_MK ? gk + j : gk;
          ra[i][j] = (mm < a.M && kq < ke) ? (A_MK ? A[int64_t(mm) * a.lda + kq] : A[int64_t(kq) * a.lda + mm]) : 0.0f;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int q = (tid + 256 * i) * VB;
      const int n = q % BN, kk = q / BN;
      const int gn = n0 + n, gk = k0 + kk;
      const TB* p = reinterpret_cast<const TB*>(a.B) + int64_t(gk) * a.ldb + gn;
      if (gk < ke && gn + VB <= a.N) {
        Vec16<TB>::load(p, rb[i]);
      } else {
#pragma unroll
        for (int j = 0; j < VB; ++j) rb[i][j] = (gk < ke && gn + j < a.N) ? Elem<TB>::load(p + j) : 0.0f;
      }
    }
  };
  f32x4_t acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  if (kb < ke) gload(kb);
  for (int k0 = kb; k0 < ke; k0 += BK) {
    __syncthreads();  // the previous chunk's reads are done
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      int m, kk;
      a_pos(i, m, kk);
      if (A_MK) {
#pragma unroll
        for (int j = 0; j < 4; ++j) As[(kk + j) * PA + m] = ra[i][j];
      } else {
        *reinterpret_cast<float4*>(&As[kk * PA + m]) = make_float4(ra[i][0], ra[i][1], ra[i][2], ra[i][3]);
      }
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int q = (tid + 256 * i) * VB;
      float* d = &Bs[(q / BN) * PB + q % BN];
#pragma unroll
      for (int j = 0; j < VB; j += 4) *reinterpret_cast<float4*>(d + j) = make_float4(rb[i][j], rb[i][j + 1], rb[i][j + 2], rb[i][j + 3]);
    }
    __syncthreads();
    if (k0 + BK < ke) gload(k0 + BK);
    // A fragment: lane holds A(m = l % 16, k = l / 16); B: B(k = l / 16, n = l % 16)
#pragma unroll
    for (int k4 = 0; k4 < BK / 4; ++k4) {
      const int kr = 4 * k4 + lane / 16;
      float af[2], bf[4];
#pragma unroll
      for (int i = 0; i < 2; ++i) af[i] = As[kr * PA + wm * 32 + i * 16 + lane % 16];
#pragma unroll
      for (int j = 0; j < 4; ++j) bf[j] = Bs[kr * PB + wn * 64 + j * 16 + lane % 16];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
  }
  rgemm_epilogue<TC, EPI>(a, acc, Cs, m0, n0, wm, wn, wave, lane);
}

// bf16-activation variant on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16):
// both operands are rounded to bf16 once (round to nearest even; x already
// is bf16), the products are accumulated in fp32. Same tiling, chunking,
// index maps and epilogues as rgemm_kernel. A fragment holds 8 consecutive
// K values of one row (A) or column (B): a K-contiguous tile ([m][k], A when
// A_MK) is read as 16 bytes per lane; tiles kept in their source orientation
// ([k][m], [k][n]) are read with the LDS transpose read ds_read_b64_tr_b16,
// which gives lane i of a 16-lane group, slot j, element i % 4 of the 8 bytes
// addressed by lane 4 j + i / 4 (so every tile store is 8 or 16 bytes wide).
typedef short rg_s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 rg_read_tr16(const bf16_t* p) {
  return __builtin_bit_cast(
      u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) rg_s16x4*)(void*)p));
}
// fragment of columns c0 .. c0 + 16 of a [k][col] tile with pitch P (elements)
__device__ __forceinline__ bf16x8_t rg_frag_tr(const bf16_t* tile, int P, int c0, int lane) {
  const int s16 = lane % 16;
  const bf16_t* p = tile + (8 * (lane / 16) + s16 / 4) * P + c0 + 4 * (s16 % 4);
  const u32x2 lo = rg_read_tr16(p), hi = rg_read_tr16(p + 4 * P);
  return __builtin_bit_cast(bf16x8_t, u32x4{lo[0], lo[1], hi[0], hi[1]});
}
__device__ __forceinline__ uint32_t rg_pack2(float a, float b) {
  return uint32_t(f32_to_bf16(a)) | (uint32_t(f32_to_bf16(b)) << 16);
}

template <typename TB, bool A_MK, typename TC, int EPI>
__global__ __launch_bounds__(256) void rgemm_bf16_kernel(VArgs a) {
  constexpr int BM = kRgBM, BN = kRgBN, BK = kRgBK;
  constexpr int PK = BK + 8;                // [m][k] pitch (bf16): 80 bytes
  constexpr int PM = BM + 8, PN = BN + 8;   // [k][m], [k][n] pitches: 144, 272 bytes
  constexpr int VB = 16 / int(sizeof(TB));  // B elements per 16-byte load
  constexpr int NA = BM * BK / 4 / 256;
  constexpr int NB = BN * BK / VB / 256;
  __shared__ __attribute__((aligned(16))) bf16_t As[A_MK ? BM * PK : BK * PM];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[BK * PN];  // [k][n]
  __shared__ __attribute__((aligned(16))) float Cs[EPI == VEPI_ADD_ACT ? 4 * 16 * (64 + 4) : 4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int kb = blockIdx.z * a.kchunk;
  const int ke = min(a.K, kb + a.kchunk);
  const float* A = reinterpret_cast<const float*>(a.A);
  const bool a_vec = (a.lda & 3) == 0 && (!A_MK || (a.kchunk & 3) == 0);
  auto a_pos = [&](int i, int& m, int& kk) {
    const int q = (tid + 256 * i) * 4;
    if (A_MK) { m = q / BK; kk = q % BK; } else { kk = q / BM; m = q % BM; }
  };
  float ra[NA][4], rb[NB][VB];
  auto gload = [&](int k0) {
    // a chunk inside M, N and the K range (uniform over the workgroup):
    // every load unconditional, so they all go out together; under the
    // per-load bounds branches below each one was waited for alone
    if (a_vec && m0 + BM <= a.M && n0 + BN <= a.N && k0 + BK <= ke) {
#pragma unroll
      for (int i = 0; i < NA; ++i) {
        int m, kk;
        a_pos(i, m, kk);
        const float4 v = *reinterpret_cast<const float4*>(A_MK ? A + int64_t(m0 + m) * a.lda + k0 + kk
                                                                : A + int64_t(k0 + kk) * a.lda + m0 + m);
        ra[i][0] = v.x; ra[i][1] = v.y; ra[i][2] = v.z; ra[i][3] = v.w;
      }
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int q = (tid + 256 * i) * VB;
        Vec16<TB>::load(reinterpret_cast<const TB*>(a.B) + int64_t(k0 + q / BN) * a.ldb + n0 + q % BN, rb[i]);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      int m, kk;
      a_pos(i, m, kk);
      const int gm = m0 + m, gk = k0 + kk;
      const bool full = A_MK ? (gm < a.M && gk + 4 <= ke) : (gk < ke && gm + 4 <= a.M);
      if (full && a_vec) {
        const float4 v = *reinterpret_cast<const float4*>(A_MK ? A + int64_t(gm) * a.lda + gk
                                                                : A + int64_t(gk) * a.lda + gm);
        ra[i][0] = v.x; ra[i][1] = v.y; ra[i][2] = v.z; ra[i][3] = v.w;
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int mm = A_MK ? gm : gm + j, kq = A_MK ? gk + j : gk;
          ra[i][j] = (mm < a.M && kq < ke) ? (A_MK ? A[int64_t(mm) * a.lda + kq] : A[int64_t(kq) * a.lda + mm]) : 0.0f;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int q = (tid + 256 * i) * VB;
      const int n = q % BN, kk = q / BN;
      const int gn = n0 + n, gk = k0 + kk;
      const TB* p = reinterpret_cast<const TB*>(a.B) + int64_t(gk) * a.ldb + gn;
      if (gk < ke && gn + VB <= a.N) {
        Vec16<TB>::load(p, rb[i]);
      } else {
#pragma unroll
        for (int j = 0; j < VB; ++j) rb[i][j] = (gk < ke && gn + j < a.N) ? Elem<TB>::load(p + j) : 0.0f;
      }
    }
  };
  f32x4_t acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  if (kb < ke) gload(kb);
  for (int k0 = kb; k0 < ke; k0 += BK) {
    __syncthreads();  // the previous chunk's reads are done
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      int m, kk;
      a_pos(i, m, kk);
      // 4 values along A's contiguous index: k ([m][k] tile) or m ([k][m] tile)
      const uint2 v = make_uint2(rg_pack2(ra[i][0], ra[i][1]), rg_pack2(ra[i][2], ra[i][3]));
      *reinterpret_cast<uint2*>(&As[A_MK ? m * PK + kk : kk * PM + m]) = v;
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int q = (tid + 256 * i) * VB;
      bf16_t* d = &Bs[(q / BN) * PN + q % BN];
      if constexpr (VB == 8) {
        *reinterpret_cast<uint4*>(d) = make_uint4(rg_pack2(rb[i][0], rb[i][1]), rg_pack2(rb[i][2], rb[i][3]),
                                                  rg_pack2(rb[i][4], rb[i][5]), rg_pack2(rb[i][6], rb[i][7]));
      } else {
        *reinterpret_cast<uint2*>(d) = make_uint2(rg_pack2(rb[i][0], rb[i][1]), rg_pack2(rb[i][2], rb[i][3]));
      }
    }
    __syncthreads();
    if (k0 + BK < ke) gload(k0 + BK);
    // fragments: lane holds row / column l % 16, K values 8 (l / 16) .. + 8
    bf16x8_t af[2], bf[4];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if constexpr (A_MK)
        af[i] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4*>(
                                                 &As[(wm * 32 + i * 16 + lane % 16) * PK + 8 * (lane / 16)]));
      else
        af[i] = rg_frag_tr(As, PM, wm * 32 + i * 16, lane);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) bf[j] = rg_frag_tr(Bs, PN, wn * 64 + j * 16, lane);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
  }
  rgemm_epilogue<TC, EPI>(a, acc, Cs, m0, n0, wm, wn, wave, lane);
}

// out[i] = sum_z part[z][i] for z = 0..Z-1 in order (deterministic).
__global__ __launch_bounds__(256) void reduce_parts_kernel(const float* __restrict__ part,
                                                           float* __restrict__ out, int64_t n, int Z) {
  for (int64_t i = blockIdx.x * int64_t(256) + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256) {
    float s = part[i];
    for (int z = 1; z < Z; ++z) s += part[z * n + i];
    out[i] = s;
  }
}

// BF16: bf16 matrix cores (bf16 activations), else fp32 matrix cores
template <bool BF16, typename TB, bool A_MK, typename TC, int EPI>
static void launch_rgemm(VArgs a, hipStream_t st, int zsplit = 1) {
  a.kchunk = (a.K + zsplit - 1) / zsplit;
  dim3 grid((a.N + kRgBN - 1) / kRgBN, (a.M + kRgBM - 1) / kRgBM, zsplit);
  if constexpr (BF16)
    rgemm_bf16_kernel<TB, A_MK, TC, EPI><<<grid, 256, 0, st>>>(a);
  else
    rgemm_kernel<TB, A_MK, TC, EPI><<<grid, 256, 0, st>>>(a);
}

// ---------------------------------------------------------------------------
// Router logits L[t][e] = (sum_i x[t][i] w[e][i]) + bias[e], each output its
// own fp32 FMA recurrence over i = 0 .. d-1 in ascending order (the same
// order everywhere, so results are bit-identical), built for latency
// hiding at low occupancy: a block holds 64 tokens x 64 experts, a thread
// 4 x 4 independent recurrences; LDS rows are K-contiguous (pitch 36 floats)
// and read 4 hidden values at a time; the next 32-wide hidden chunk is
// fetched with 16-byte global loads into registers while the current one is
// consumed, and LDS is double-buffered. Expert rows are interleaved by 16
// across lanes (thread tn owns experts tn + 16 j), which makes the float4
// reads of the weight tile conflict-free; token rows are shared by 16 lanes
// (broadcast). d must be a multiple of 32.
// ---------------------------------------------------------------------------
constexpr int kLgTM = 64, kLgKC = 32, kLgP = kLgKC + 4;

// Clears n ints of p (nothing when p is null), spread over the whole grid:
// the logits kernels clear the fused route-and-dispatch histogram this way,
// so that the selection kernel, next on the stream, can count into it.
__device__ __forceinline__ void clear_grid_part(int32_t* p, int64_t n) {
  if (!p) return;
  const int64_t nb = int64_t(gridDim.x) * gridDim.y;
  const int64_t b = int64_t(blockIdx.y) * gridDim.x + blockIdx.x;
  for (int64_t i = b * 256 + threadIdx.x; i < n; i += nb * 256) p[i] = 0;
}

// TN = 64 experts per block, or 32 when 64 would leave fewer than two blocks
// per CU (then a thread holds 4 x 2 recurrences)
template <typename TX, int TN>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void logits_kernel(const TX* __restrict__ x, const float* __restrict__ w,
                                                     const float* __restrict__ bias, float* __restrict__ out,
                                                     int T, int E, int d, int32_t* clr, int64_t nclr) {
  clear_grid_part(clr, nclr);
  constexpr int FN = TN / 16;                  // expert columns per thread
  constexpr int WL = TN * kLgKC / 4 / 256;     // w loads per thread
  __shared__ __attribute__((aligned(16))) float As[2][kLgTM * kLgP];
  __shared__ __attribute__((aligned(16))) float Bs[2][TN * kLgP];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.y * kLgTM, e0 = blockIdx.x * TN;
  const int tm = tid / 16, tn = tid % 16;
  // global -> register plan. x chunk: 64 rows x 32 values; w chunk: 64 rows x 32 floats
  constexpr int XV = 16 / sizeof(TX);              // x values per 16-byte load
  constexpr int XL = kLgTM * kLgKC / XV / 256;     // x loads per thread (1 bf16, 2 f32)
  int xrow[XL], xk[XL];
#pragma unroll
  for (int q = 0; q < XL; ++q) {
    const int idx = tid + 256 * q;
    xrow[q] = idx / (kLgKC / XV);
    xk[q] = (idx % (kLgKC / XV)) * XV;
  }
  int wrow[WL], wk[WL];
#pragma unroll
  for (int q = 0; q < WL; ++q) {
    const int idx = tid + 256 * q;
    wrow[q] = idx / (kLgKC / 4);
    wk[q] = (idx % (kLgKC / 4)) * 4;
  }
  const int nch = d / kLgKC;
  // A chunk's loads go out with no branch around them and stay raw until
  // the next chunk has been computed: rows past T (experts past E) read
  // the last one, in bounds, and are zeroed when stored to LDS. (Converted
  // under a bounds branch, each load was waited for as soon as issued.)
  uint4 xraw[XL];
  float4 wv[WL];
  auto gload = [&](int c) {
    const int k0 = c * kLgKC;
#pragma unroll
    for (int q = 0; q < XL; ++q)
      xraw[q] = *reinterpret_cast<const uint4*>(x + int64_t(min(t0 + xrow[q], T - 1)) * d + k0 + xk[q]);
#pragma unroll
    for (int q = 0; q < WL; ++q)
      wv[q] = *reinterpret_cast<const float4*>(w + int64_t(min(e0 + wrow[q], E - 1)) * d + k0 + wk[q]);
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int q = 0; q < XL; ++q) {
      float xv[XV];
      Vec16<TX>::unpack(xraw[q], xv);
      const bool in = t0 + xrow[q] < T;
#pragma unroll
      for (int v = 0; v < XV; v += 4)
        *reinterpret_cast<float4*>(&As[buf][xrow[q] * kLgP + xk[q] + v]) =
            in ? make_float4(xv[v], xv[v + 1], xv[v + 2], xv[v + 3]) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
#pragma unroll
    for (int q = 0; q < WL; ++q)
      *reinterpret_cast<float4*>(&Bs[buf][wrow[q] * kLgP + wk[q]]) =
          e0 + wrow[q] < E ? wv[q] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  };
  float acc[4][FN];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = 0.0f;
  auto compute = [&](int buf) {
#pragma unroll 2
    for (int k = 0; k < kLgKC; k += 4) {
      float4 a[4], b[FN];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const float4*>(&As[buf][(tm + 16 * i) * kLgP + k]);
#pragma unroll
      for (int j = 0; j < FN; ++j) b[j] = *reinterpret_cast<const float4*>(&Bs[buf][(tn + 16 * j) * kLgP + k]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          acc[i][j] = __builtin_fmaf(a[i].x, b[j].x, acc[i][j]);
          acc[i][j] = __builtin_fmaf(a[i].y, b[j].y, acc[i][j]);
          acc[i][j] = __builtin_fmaf(a[i].z, b[j].z, acc[i][j]);
          acc[i][j] = __builtin_fmaf(a[i].w, b[j].w, acc[i][j]);
        }
    }
  };
  gload(0);
  lstore(0);
  __syncthreads();
  for (int c = 0; c + 1 < nch; ++c) {
    gload(c + 1);
    compute(c & 1);
    lstore((c + 1) & 1);
    __syncthreads();
  }
  compute((nch - 1) & 1);
  float bv[FN];  // this lane's experts' biases, loaded together
#pragma unroll
  for (int j = 0; j < FN; ++j) bv[j] = bias ? bias[min(e0 + tn + 16 * j, E - 1)] : 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + tm + 16 * i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int e = e0 + tn + 16 * j;
      if (e >= E) continue;
      float v = acc[i][j];
      if (bias) v = v + bv[j];
      out[int64_t(t) * E + e] = v;
    }
  }
}

// Router logits for few experts (E <= 32): one thread per (token, expert)
// recurrence, same ascending order. A block holds 256 / EP tokens x EP
// experts (EP = E rounded up to a power of two); the 256-wide hidden chunk
// of the block's tokens and of all experts' weights is staged in LDS
// (16-byte global loads, prefetched into registers, double-buffered LDS) and
// read 4 hidden values at a time; token rows are shared by the EP lanes of a
// token and weight rows by the tokens of a wave (broadcast reads). A chunk is
// long enough (256 dependent FMAs per lane) to cover the next chunk's load
// latency. d must be a multiple of 4; the last chunk may be partial.
constexpr int kSeKC = 256, kSeP = kSeKC + 4;

template <typename TX, int EP>
__global__ __launch_bounds__(256) void logits_small_e_kernel(const TX* __restrict__ x, const float* __restrict__ w,
                                                             const float* __restrict__ bias, float* __restrict__ out,
                                                             int T, int E, int d, int32_t* clr, int64_t nclr) {
  clear_grid_part(clr, nclr);
  constexpr int TPB = 256 / EP;  // tokens per block
  __shared__ __attribute__((aligned(16))) float Xs[2][TPB * kSeP];
  __shared__ __attribute__((aligned(16))) float Ws[2][EP * kSeP];
  const int tid = threadIdx.x;
  const int e = tid % EP, tl = tid / EP;
  const int t0 = blockIdx.x * TPB;
  // x chunk: TPB rows x 64 values; w chunk: EP rows x 64 floats
  constexpr int XV = 16 / sizeof(TX);
  constexpr int XU = TPB * kSeKC / XV;   // 16-byte units of the x chunk
  constexpr int WU = EP * kSeKC / 4;     // 16-byte units of the w chunk
  constexpr int XL = (XU + 255) / 256, WL = (WU + 255) / 256;
  const int nch = (d + kSeKC - 1) / kSeKC;
  static_assert(XU % 256 == 0 && WU % 256 == 0, "whole load rounds");
  // A chunk's loads go out with no branch around them and stay raw until
  // the next chunk has been computed: a unit past T, E or d reads the last
  // row / chunk in bounds and is zeroed when stored to LDS. (Converted
  // under a bounds branch, each load was waited for as soon as issued.)
  uint4 xraw[XL];
  float4 wv[WL];
  bool xin[XL], win[WL];
  auto gload = [&](int c) {
    const int k0 = c * kSeKC;
#pragma unroll
    for (int q = 0; q < XL; ++q) {
      const int u = tid + 256 * q, r = u / (kSeKC / XV), kk = (u % (kSeKC / XV)) * XV;
      xin[q] = t0 + r < T && k0 + kk < d;
      xraw[q] = *reinterpret_cast<const uint4*>(x + int64_t(min(t0 + r, T - 1)) * d + min(k0 + kk, d - XV));
    }
#pragma unroll
    for (int q = 0; q < WL; ++q) {
      const int u = tid + 256 * q, r = u / (kSeKC / 4), kk = (u % (kSeKC / 4)) * 4;
      win[q] = r < E && k0 + kk < d;
      wv[q] = *reinterpret_cast<const float4*>(w + int64_t(min(r, E - 1)) * d + min(k0 + kk, d - 4));
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int q = 0; q < XL; ++q) {
      const int u = tid + 256 * q, r = u / (kSeKC / XV), kk = (u % (kSeKC / XV)) * XV;
      float xv[XV];
      Vec16<TX>::unpack(xraw[q], xv);
#pragma unroll
      for (int v = 0; v < XV; v += 4)
        *reinterpret_cast<float4*>(&Xs[buf][r * kSeP + kk + v]) =
            xin[q] ? make_float4(xv[v], xv[v + 1], xv[v + 2], xv[v + 3]) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
#pragma unroll
    for (int q = 0; q < WL; ++q) {
      const int u = tid + 256 * q, r = u / (kSeKC / 4), kk = (u % (kSeKC / 4)) * 4;
      *reinterpret_cast<float4*>(&Ws[buf][r * kSeP + kk]) = win[q] ? wv[q] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
  };
  float acc = 0.0f;
  auto compute = [&](int buf, int kend) {
#pragma unroll 4
    for (int k = 0; k < kend; k += 4) {
      const float4 a = *reinterpret_cast<const float4*>(&Xs[buf][tl * kSeP + k]);
      const float4 b = *reinterpret_cast<const float4*>(&Ws[buf][e * kSeP + k]);
      acc = __builtin_fmaf(a.x, b.x, acc);
      acc = __builtin_fmaf(a.y, b.y, acc);
      acc = __builtin_fmaf(a.z, b.z, acc);
      acc = __builtin_fmaf(a.w, b.w, acc);
    }
  };
  gload(0);
  lstore(0);
  __syncthreads();
  for (int c = 0; c + 1 < nch; ++c) {
    gload(c + 1);
    compute(c & 1, kSeKC);
    lstore((c + 1) & 1);
    __syncthreads();
  }
  compute((nch - 1) & 1, d - (nch - 1) * kSeKC);
  const int t = t0 + tl;
  if (t < T && e < E) {
    float v = acc;
    if (bias) v = v + bias[e];
    out[int64_t(t) * E + e] = v;
  }
}

template <typename TX>
static void launch_logits_small_e(const RouteLaunch& r, hipStream_t st) {
  const TX* x = reinterpret_cast<const TX*>(r.x);
  const int T = int(r.T), E = int(r.E), d = int(r.d);
  const int64_t nclr = r.chunk_cnt ? (r.T + kChunkTok - 1) / kChunkTok * r.E : 0;
  auto grid = [&](int ep) { return dim3(unsigned((T + 256 / ep - 1) / (256 / ep))); };
  if (E <= 8)
    logits_small_e_kernel<TX, 8><<<grid(8), 256, 0, st>>>(x, r.w_router, r.bias, r.logits, T, E, d, r.chunk_cnt, nclr);
  else if (E <= 16)
    logits_small_e_kernel<TX, 16><<<grid(16), 256, 0, st>>>(x, r.w_router, r.bias, r.logits, T, E, d, r.chunk_cnt, nclr);
  else
    logits_small_e_kernel<TX, 32><<<grid(32), 256, 0, st>>>(x, r.w_router, r.bias, r.logits, T, E, d, r.chunk_cnt, nclr);
}

// Token-chunk count of the router weight gradient: enough workgroups to
// fill the chip, chunks of at least 128 tokens.
int route_bwd_zsplit(int64_t T, int64_t d, int64_t E) {
  const int64_t base = ((d + kRgBN - 1) / kRgBN) * ((E + kRgBM - 1) / kRgBM);
  int64_t z = (1024 + base - 1) / base;
  z = z < 1 ? 1 : z;
  const int64_t zmax = (T + 255) / 256;
  if (z > zmax) z = zmax < 1 ? 1 : zmax;
  return int(z);
}

// ---------------------------------------------------------------------------
// Selection: one wave per token. 64-bit keys (ordered logit << 32 | ~expert)
// make "larger logit first, lower expert on ties" a plain unsigned maximum.
// -0 is folded into +0; NaN maps below every number; 0 means "not eligible".
// ---------------------------------------------------------------------------
constexpr int kMaxK = 16;

__device__ __forceinline__ uint64_t make_key(float L, int e) {
  uint32_t u = __float_as_uint(L);
  uint32_t ord;
  if (L != L) ord = 0u;
  else {
    if (u == 0x80000000u) u = 0u;
    ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  }
  return (uint64_t(ord) << 32) | uint64_t(0xFFFFFFFFu - uint32_t(e));
}

__device__ __forceinline__ float key_logit(uint64_t key) {
  const uint32_t ord = uint32_t(key >> 32);
  const uint32_t u = (ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord;
  return __uint_as_float(u);
}

__device__ __forceinline__ int key_expert(uint64_t key) {
  return int(0xFFFFFFFFu - uint32_t(key));
}

// (Sa, a) strictly above (Sb, b): larger first, NaN last, then lower index.
__device__ __forceinline__ bool score_above(float Sa, int a, float Sb, int b) {
  const bool na = Sa != Sa, nb = Sb != Sb;
  if (na != nb) return nb;
  if (!na && Sa != Sb) return Sa > Sb;
  return a < b;
}

struct SelArgs {
  const float* logits;
  int T, E, k;
  int score_fn, renorm;
  float gate_scale;
  int num_groups, topk_groups, group_score;
  int32_t* idx;
  float* gate;
  uint8_t* rmap;
  int32_t* chunk_cnt;  // or null: the per-chunk expert histogram of the fused route and dispatch
};

template <int NPL>
__global__ __launch_bounds__(256) void select_kernel(SelArgs s) {
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int t = blockIdx.x * 4 + wave;
  if (t >= s.T) return;
  const float* Lrow = s.logits + int64_t(t) * s.E;

  uint64_t key[NPL];
  float Lv[NPL];
  // every load of the row at once (a lane past E reads the last logit, in
  // bounds, and drops it): under a bounds branch each was waited for alone
#pragma unroll
  for (int p = 0; p < NPL; ++p) Lv[p] = Lrow[min(lane + kWave * p, s.E - 1)];
#pragma unroll
  for (int p = 0; p < NPL; ++p) {
    const int e = lane + kWave * p;
    Lv[p] = e < s.E ? Lv[p] : 0.0f;
    key[p] = e < s.E ? make_key(Lv[p], e) : 0;
  }
  // global best logit (softmax normaliser), before any group masking
  uint64_t gbest = 0;
#pragma unroll
  for (int p = 0; p < NPL; ++p) gbest = key[p] > gbest ? key[p] : gbest;
  gbest = wave_max_u64(gbest);

  if (s.num_groups > 1 && s.topk_groups < s.num_groups) {
    const int gs = s.E / s.num_groups;
    float my_gscore = 0.0f;  // lane g holds the score of group g
    for (int g = 0; g < s.num_groups; ++g) {
      uint64_t m1 = 0;
#pragma unroll
      for (int p = 0; p < NPL; ++p) {
        const int e = lane + kWave * p;
        if (e < s.E && e / gs == g && key[p] > m1) m1 = key[p];
      }
      m1 = wave_max_u64(m1);
      uint64_t m2 = 0;
#pragma unroll
      for (int p = 0; p < NPL; ++p) {
        const int e = lane + kWave * p;
        if (e < s.E && e / gs == g && key[p] != m1 && key[p] > m2) m2 = key[p];
      }
      m2 = wave_max_u64(m2);
      float sc = sigmoid_spec(key_logit(m1));
      if (s.group_score == 0 && gs > 1) sc = sc + sigmoid_spec(key_logit(m2));
      if (lane == g) my_gscore = sc;
    }
    // keep the topk_groups best groups: larger score first, lower group on ties
    uint32_t kept = 0;
    for (int r = 0; r < s.topk_groups; ++r) {
      uint64_t gk = (lane < s.num_groups && !((kept >> lane) & 1u)) ? make_key(my_gscore, lane) : 0;
      gk = wave_max_u64(gk);
      kept |= 1u << key_expert(gk);
    }
#pragma unroll
    for (int p = 0; p < NPL; ++p) {
      const int e = lane + kWave * p;
      if (e < s.E && !((kept >> (e / gs)) & 1u)) key[p] = 0;
    }
  }

  int sel_e[kMaxK];
  float sel_L[kMaxK];
  uint32_t mine = 0;  // bit p set: expert lane + 64p was selected
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j < s.k) {
      uint64_t m = 0;
#pragma unroll
      for (int p = 0; p < NPL; ++p) m = key[p] > m ? key[p] : m;
      m = wave_max_u64(m);
      sel_e[j] = key_expert(m);
      sel_L[j] = key_logit(m);
#pragma unroll
      for (int p = 0; p < NPL; ++p)
        if (key[p] == m) {
          key[p] = 0;
          mine |= 1u << p;
        }
    } else {
      sel_e[j] = 0;
      sel_L[j] = 0.0f;
    }
  }

  // gates
  float g[kMaxK];
  if (s.score_fn == 0) {  // softmax
    if (s.renorm) {
      const float m = sel_L[0];
      float Z = 0.0f;
#pragma unroll
      for (int j = 0; j < kMaxK; ++j) {
        g[j] = (j < s.k) ? exp_spec(sel_L[j] - m) : 0.0f;
        Z = Z + g[j];
      }
#pragma unroll
      for (int j = 0; j < kMaxK; ++j) g[j] = g[j] / Z * s.gate_scale;
    } else {
      const float m = key_logit(gbest);
      float z = 0.0f;
#pragma unroll
      for (int p = 0; p < NPL; ++p)
        if (lane + kWave * p < s.E) z += exp_spec(Lv[p] - m);
      const float Z = wave_sum(z);
#pragma unroll
      for (int j = 0; j < kMaxK; ++j)
        g[j] = (j < s.k) ? exp_spec(sel_L[j] - m) / Z * s.gate_scale : 0.0f;
    }
  } else {  // sigmoid
    float Z = 0.0f;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      g[j] = (j < s.k) ? sigmoid_spec(sel_L[j]) : 0.0f;
      Z = Z + g[j];
    }
#pragma unroll
    for (int j = 0; j < kMaxK; ++j)
      g[j] = s.renorm ? g[j] / Z * s.gate_scale : g[j] * s.gate_scale;
  }

#pragma unroll
  for (int j = 0; j < kMaxK; ++j)
    if (j < s.k && lane == j) {
      s.idx[int64_t(t) * s.k + j] = sel_e[j];
      s.gate[int64_t(t) * s.k + j] = g[j];
    }
  if (s.chunk_cnt) {
    // the dispatch histogram, fused into the selection: lane j < k adds the
    // token's j-th expert to its chunk's count (integer atomics: the result
    // does not depend on their order; the logits kernel cleared the counts)
    int mine_e = 0;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j)
      if (lane == j) mine_e = sel_e[j];
    if (lane < s.k) atomicAdd(&s.chunk_cnt[int64_t(t / kChunkTok) * s.E + mine_e], 1);
  }
  if (s.rmap) {
#pragma unroll
    for (int p = 0; p < NPL; ++p) {
      const int e = lane + kWave * p;
      if (e < s.E) s.rmap[int64_t(t) * s.E + e] = (mine >> p) & 1u;
    }
  }
}

// ---------------------------------------------------------------------------
// Router backward, first step: dL [T,E] from d_gate, one wave per token.
// ---------------------------------------------------------------------------
struct DLArgs {
  const float* logits;
  const int32_t* idx;
  const float* dgate;
  float* dL;
  int T, E, k;
  int score_fn, renorm;
  float gate_scale;
  // auxiliary loss (aux_f NULL: off): f [E] and the upstream gradient d_aux
  // [1]; aux_scale = coeff * E / T
  const float* aux_f;
  const float* d_aux;
  float aux_scale;
};

template <int NPL>
__global__ __launch_bounds__(256) void dlogits_kernel(DLArgs a) {
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int t = blockIdx.x * 4 + wave;
  if (t >= a.T) return;
  const float* Lrow = a.logits + int64_t(t) * a.E;
  float dl[NPL];
#pragma unroll
  for (int p = 0; p < NPL; ++p) dl[p] = 0.0f;
  int e_j[kMaxK];
  float L_j[kMaxK], dg_j[kMaxK];
  // all k slots' loads in two rounds (indices and gate gradients, then the
  // selected logits); slots past k read slot k - 1, in bounds, and are
  // dropped. Under a per-slot branch each load was waited for alone.
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    const int64_t o = int64_t(t) * a.k + min(j, a.k - 1);
    e_j[j] = a.idx[o];
    dg_j[j] = a.dgate[o];
  }
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) L_j[j] = Lrow[e_j[j]];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    e_j[j] = j < a.k ? e_j[j] : -1;
    L_j[j] = j < a.k ? L_j[j] : 0.0f;
    dg_j[j] = j < a.k ? dg_j[j] : 0.0f;
  }
  const float c = a.gate_scale;
  float sel_grad[kMaxK];  // dL for each selected slot (sparse rules)
  bool dense = false;
  if (a.score_fn == 0 && a.renorm) {
    float m = L_j[0];
#pragma unroll
    for (int j = 1; j < kMaxK; ++j)
      if (j < a.k) m = fmaxf(m, L_j[j]);
    float q[kMaxK], Z = 0.0f;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      q[j] = (j < a.k) ? expf(L_j[j] - m) : 0.0f;
      Z += q[j];
    }
    float S = 0.0f;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      q[j] /= Z;
      S += q[j] * dg_j[j];
    }
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) sel_grad[j] = c * q[j] * (dg_j[j] - S);
  } else if (a.score_fn == 0) {
    dense = true;
    float Lv[NPL];
    float m = -__builtin_inff();
#pragma unroll
    for (int p = 0; p < NPL; ++p) {
      const int e = lane + kWave * p;
      Lv[p] = e < a.E ? Lrow[e] : -__builtin_inff();
      m = fmaxf(m, Lv[p]);
    }
    m = wave_max(m);
    float z = 0.0f;
#pragma unroll
    for (int p = 0; p < NPL; ++p)
      if (lane + kWave * p < a.E) z += expf(Lv[p] - m);
    const float Z = wave_sum(z);
    float S = 0.0f;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j)
      if (j < a.k) S += expf(L_j[j] - m) / Z * dg_j[j];
#pragma unroll
    for (int p = 0; p < NPL; ++p) {
      const int e = lane + kWave * p;
      if (e >= a.E) continue;
      float dhat = 0.0f;
#pragma unroll
      for (int j = 0; j < kMaxK; ++j)
        if (j < a.k && e_j[j] == e) dhat = dg_j[j];
      const float pe = expf(Lv[p] - m) / Z;
      dl[p] = c * pe * (dhat - S);
    }
  } else {
    float s[kMaxK], Z = 0.0f, S = 0.0f;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      s[j] = (j < a.k) ? 1.0f / (1.0f + expf(-L_j[j])) : 0.0f;
      Z += s[j];
      S += dg_j[j] * s[j];
    }
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      const float ds = a.renorm ? c * (dg_j[j] / Z - S / (Z * Z)) : c * dg_j[j];
      sel_grad[j] = ds * s[j] * (1.0f - s[j]);
    }
  }
  if (!dense) {
#pragma unroll
    for (int p = 0; p < NPL; ++p) {
      const int e = lane + kWave * p;
#pragma unroll
      for (int j = 0; j < kMaxK; ++j)
        if (j < a.k && e_j[j] == e) dl[p] = sel_grad[j];
    }
  }
  if (a.aux_f) {
    // + aux_scale * d_aux * p_e * (f_e - sum_j f_j p_j), p the softmax over
    // all experts
    float Lv[NPL], fv[NPL];
    float m = -__builtin_inff();
#pragma unroll
    for (int p = 0; p < NPL; ++p) {
      const int e = lane + kWave * p;
      Lv[p] = e < a.E ? Lrow[e] : -__builtin_inff();
      fv[p] = e < a.E ? a.aux_f[e] : 0.0f;
      m = fmaxf(m, Lv[p]);
    }
    m = wave_max(m);
    float q[NPL], z = 0.0f;
#pragma unroll
    for (int p = 0; p < NPL; ++p) {
      q[p] = lane + kWave * p < a.E ? expf(Lv[p] - m) : 0.0f;
      z += q[p];
    }
    const float Z = wave_sum(z);
    float dot = 0.0f;
#pragma unroll
    for (int p = 0; p < NPL; ++p) {
      q[p] /= Z;
      dot += fv[p] * q[p];
    }
    dot = wave_sum(dot);
    const float sc = a.aux_scale * a.d_aux[0];
#pragma unroll
    for (int p = 0; p < NPL; ++p) dl[p] += sc * q[p] * (fv[p] - dot);
  }
#pragma unroll
  for (int p = 0; p < NPL; ++p) {
    const int e = lane + kWave * p;
    if (e < a.E) a.dL[int64_t(t) * a.E + e] = dl[p];
  }
}

// ---------------------------------------------------------------------------
// Load-balancing auxiliary loss (Switch form, see moe_route_aux_loss):
//   aux_partials_kernel  one block per chunk of tokens: the chunk's expert
//                        counts (LDS integer histogram) and, with WITH_P, its
//                        sum of softmax probabilities (one wave per token,
//                        each wave loading several rows before reducing any,
//                        waves added in wave order);
//   aux_final_kernel     one block: adds the chunk partials in chunk order,
//                        writes f_e = count_e / (T k) and/or the loss.
// Integer counts are exact; the float sums have a fixed order, so the result
// is deterministic. HBM traffic: logits once (T E 4 bytes) plus idx.
// ---------------------------------------------------------------------------
constexpr int kAuxMaxBlocks = 256;  // chunks: enough blocks for small T, few partials for large T
constexpr int kAuxWaves = 8;        // waves per block of aux_partials_kernel
constexpr int kAuxRows = 4;         // logit rows a wave loads before reducing them

static int64_t aux_tokens_per_block(int64_t T) {
  const int64_t per = (T + kAuxMaxBlocks - 1) / kAuxMaxBlocks;
  return per < 32 ? 32 : (per + 31) / 32 * 32;
}

int aux_blocks(int64_t T) {
  return T <= 0 ? 0 : int((T + aux_tokens_per_block(T) - 1) / aux_tokens_per_block(T));
}

template <int NPL, bool WITH_P>
__global__ __launch_bounds__(kAuxWaves * kWave) void aux_partials_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ idx, float* __restrict__ p_part,
    int32_t* __restrict__ c_part, int T, int E, int k, int tpb) {
  __shared__ float ps[WITH_P ? kAuxWaves : 1][kWave * NPL];
  __shared__ int cnt[kWave * NPL];
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int t0 = blockIdx.x * tpb;
  const int nt = min(tpb, T - t0);
  for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
  __syncthreads();
  const int32_t* ib = idx + int64_t(t0) * k;
  for (int i = threadIdx.x; i < nt * k; i += blockDim.x) {
    const int e = ib[i];
    if (unsigned(e) < unsigned(E)) atomicAdd(&cnt[e], 1);
  }
  if constexpr (WITH_P) {
    float acc[NPL];
#pragma unroll
    for (int p = 0; p < NPL; ++p) acc[p] = 0.0f;
    // wave w takes tokens w, w + 8, w + 16, ...: kAuxRows rows loaded at once
    for (int tt = wave; tt < nt; tt += kAuxWaves * kAuxRows) {
      float Lv[kAuxRows][NPL];
#pragma unroll
      for (int r = 0; r < kAuxRows; ++r) {
        const int t = tt + r * kAuxWaves;
        const float* Lrow = logits + int64_t(t0 + t) * E;
#pragma unroll
        for (int p = 0; p < NPL; ++p) {
          const int e = lane + kWave * p;
          Lv[r][p] = (t < nt && e < E) ? Lrow[e] : -__builtin_inff();
        }
      }
#pragma unroll
      for (int r = 0; r < kAuxRows; ++r) {
        if (tt + r * kAuxWaves >= nt) break;
        float m = Lv[r][0];
#pragma unroll
        for (int p = 1; p < NPL; ++p) m = fmaxf(m, Lv[r][p]);
        m = wave_max(m);
        float q[NPL], z = 0.0f;
#pragma unroll
        for (int p = 0; p < NPL; ++p) {
          q[p] = lane + kWave * p < E ? expf(Lv[r][p] - m) : 0.0f;
          z += q[p];
        }
        const float Z = wave_sum(z);
#pragma unroll
        for (int p = 0; p < NPL; ++p) acc[p] += q[p] / Z;
      }
    }
#pragma unroll
    for (int p = 0; p < NPL; ++p) ps[wave][lane + kWave * p] = acc[p];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    c_part[int64_t(blockIdx.x) * E + e] = cnt[e];
    if constexpr (WITH_P) {
      float v = ps[0][e];
#pragma unroll
      for (int w = 1; w < kAuxWaves; ++w) v += ps[w][e];
      p_part[int64_t(blockIdx.x) * E + e] = v;
    }
  }
}

// 1024 threads: expert e gets S = 1024 / E threads, split s adds chunks
// s, s+S, s+2S, ... in order; the S split sums are then added in split order.
// WITH_P: probability sums present (the loss); without, only f_e.
template <bool WITH_P>
__global__ __launch_bounds__(1024) void aux_final_kernel(const float* __restrict__ p_part,
                                                         const int32_t* __restrict__ c_part,
                                                         int nblk, int E, float tk,
                                                         float loss_scale, float* __restrict__ f_out,
                                                         float* __restrict__ loss) {
  __shared__ float sp[WITH_P ? 1024 : 1];
  __shared__ int sc[1024];
  __shared__ float red[WITH_P ? 1024 : 1];
  const int tid = threadIdx.x;
  const int S = 1024 / E;
  if (tid < S * E) {
    const int e = tid % E, s = tid / E;
    int c = 0;
    float P = 0.0f;
#pragma unroll 16
    for (int b = s; b < nblk; b += S) {
      c += c_part[int64_t(b) * E + e];
      if constexpr (WITH_P) P += p_part[int64_t(b) * E + e];
    }
    if constexpr (WITH_P) sp[tid] = P;
    sc[tid] = c;
  }
  __syncthreads();
  float term = 0.0f;
  if (tid < E) {
    int c = 0;
    float P = 0.0f;
    for (int s = 0; s < S; ++s) {
      c += sc[s * E + tid];
      if constexpr (WITH_P) P += sp[s * E + tid];
    }
    const float fe = float(c) / tk;
    if (f_out) f_out[tid] = fe;
    term = fe * P;
  }
  if constexpr (WITH_P) {
    red[tid] = term;
    __syncthreads();
    for (int o = 512; o > 0; o >>= 1) {
      if (tid < o) red[tid] += red[tid + o];
      __syncthreads();
    }
    if (tid == 0) loss[0] = loss_scale * red[0];
  }
}

template <bool WITH_P>
static void launch_aux_partials(const float* logits, const int32_t* idx, float* p_part,
                                int32_t* c_part, int64_t T, int64_t E, int64_t k, hipStream_t st) {
  const int nb = aux_blocks(T);
  const int tpb = int(aux_tokens_per_block(T));
  const int t = int(T), e = int(E), kk = int(k);
  constexpr int B = kAuxWaves * kWave;
  if (E <= 64) aux_partials_kernel<1, WITH_P><<<nb, B, 0, st>>>(logits, idx, p_part, c_part, t, e, kk, tpb);
  else if (E <= 128) aux_partials_kernel<2, WITH_P><<<nb, B, 0, st>>>(logits, idx, p_part, c_part, t, e, kk, tpb);
  else if (E <= 256) aux_partials_kernel<4, WITH_P><<<nb, B, 0, st>>>(logits, idx, p_part, c_part, t, e, kk, tpb);
  else if (E <= 512) aux_partials_kernel<8, WITH_P><<<nb, B, 0, st>>>(logits, idx, p_part, c_part, t, e, kk, tpb);
  else aux_partials_kernel<16, WITH_P><<<nb, B, 0, st>>>(logits, idx, p_part, c_part, t, e, kk, tpb);
}

void launch_route_aux_loss(const AuxLaunch& a, hipStream_t st) {
  launch_aux_partials<true>(a.logits, a.idx, a.p_part, a.c_part, a.T, a.E, a.k, st);
  aux_final_kernel<true><<<1, 1024, 0, st>>>(a.p_part, a.c_part, aux_blocks(a.T), int(a.E),
                                             float(a.T * a.k), a.coeff * float(a.E) / float(a.T),
                                             nullptr, a.loss);
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
template <typename TX>
static void route_fwd_t(const RouteLaunch& r, hipStream_t st) {
  if (r.E >= 32) {
    const unsigned gy = unsigned((r.T + kLgTM - 1) / kLgTM);
    const int64_t blocks64 = int64_t((r.E + 63) / 64) * gy;
    const int64_t nclr = r.chunk_cnt ? (r.T + kChunkTok - 1) / kChunkTok * r.E : 0;
    if (blocks64 >= 512)
      logits_kernel<TX, 64><<<dim3(unsigned((r.E + 63) / 64), gy), 256, 0, st>>>(
          reinterpret_cast<const TX*>(r.x), r.w_router, r.bias, r.logits, int(r.T), int(r.E), int(r.d),
          r.chunk_cnt, nclr);
    else
      logits_kernel<TX, 32><<<dim3(unsigned((r.E + 31) / 32), gy), 256, 0, st>>>(
          reinterpret_cast<const TX*>(r.x), r.w_router, r.bias, r.logits, int(r.T), int(r.E), int(r.d),
          r.chunk_cnt, nclr);
  } else {
    launch_logits_small_e<TX>(r, st);
  }

  SelArgs s{};
  s.logits = r.logits; s.T = int(r.T); s.E = int(r.E); s.k = int(r.k);
  s.score_fn = r.score_fn; s.renorm = r.renorm; s.gate_scale = r.gate_scale;
  s.num_groups = r.num_groups; s.topk_groups = r.topk_groups; s.group_score = r.group_score;
  s.idx = r.idx; s.gate = r.gate; s.rmap = r.rmap; s.chunk_cnt = r.chunk_cnt;
  const dim3 grid((r.T + 3) / 4);
  if (r.E <= 64) select_kernel<1><<<grid, 256, 0, st>>>(s);
  else if (r.E <= 128) select_kernel<2><<<grid, 256, 0, st>>>(s);
  else if (r.E <= 256) select_kernel<4><<<grid, 256, 0, st>>>(s);
  else if (r.E <= 512) select_kernel<8><<<grid, 256, 0, st>>>(s);
  else select_kernel<16><<<grid, 256, 0, st>>>(s);
}

void launch_route_fwd(const RouteLaunch& r, hipStream_t st) {
  if (r.act_bf16) route_fwd_t<bf16_t>(r, st);
  else route_fwd_t<float>(r, st);
}

template <typename TX>
static void route_bwd_t(const RouteBwdLaunch& r, hipStream_t st) {
  DLArgs d{};
  d.logits = r.logits; d.idx = r.idx; d.dgate = r.dgate; d.dL = r.dL;
  d.T = int(r.T); d.E = int(r.E); d.k = int(r.k);
  d.score_fn = r.score_fn; d.renorm = r.renorm; d.gate_scale = r.gate_scale;
  if (r.d_aux) {
    // f_e from the selection, then the aux term inside dlogits_kernel
    launch_aux_partials<false>(nullptr, r.idx, nullptr, r.aux_counts, r.T, r.E, r.k, st);
    aux_final_kernel<false><<<1, 1024, 0, st>>>(nullptr, r.aux_counts, aux_blocks(r.T), int(r.E),
                                                float(r.T * r.k), 0.0f, r.aux_f, nullptr);
    d.aux_f = r.aux_f;
    d.d_aux = r.d_aux;
    d.aux_scale = r.aux_coeff * float(r.E) / float(r.T);
  }
  const dim3 grid((r.T + 3) / 4);
  if (r.E <= 64) dlogits_kernel<1><<<grid, 256, 0, st>>>(d);
  else if (r.E <= 128) dlogits_kernel<2><<<grid, 256, 0, st>>>(d);
  else if (r.E <= 256) dlogits_kernel<4><<<grid, 256, 0, st>>>(d);
  else if (r.E <= 512) dlogits_kernel<8><<<grid, 256, 0, st>>>(d);
  else dlogits_kernel<16><<<grid, 256, 0, st>>>(d);

  // dx[t,:] += sum_e dL[t,e] w[e,:]
  VArgs v{};
  v.A = r.dL; v.lda = r.E;
  v.B = r.w_router; v.ldb = r.d;
  v.C = r.dx; v.ldc = r.d;
  v.M = int(r.T); v.N = int(r.d); v.K = int(r.E);
  constexpr bool BF16 = sizeof(TX) == 2;
  launch_rgemm<BF16, float, true, TX, VEPI_ADD_ACT>(v, st);

  // dw[e,:] = sum_t dL[t,e] x[t,:], tokens split into Z chunks whose partial
  // sums are added in chunk order
  const int Z = route_bwd_zsplit(r.T, r.d, r.E);
  VArgs w{};
  w.A = r.dL; w.lda = r.E;
  w.B = r.x; w.ldb = r.d;
  w.C = Z > 1 ? r.dw_part : r.dw_router; w.ldc = r.d;
  w.c_zstride = r.E * r.d;
  w.M = int(r.E); w.N = int(r.d); w.K = int(r.T);
  launch_rgemm<BF16, TX, false, float, VEPI_STORE>(w, st, Z);
  if (Z > 1) {
    const int64_t n = r.E * r.d;
    reduce_parts_kernel<<<int((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096), 256, 0, st>>>(
        r.dw_part, r.dw_router, n, Z);
  }
}

void launch_route_bwd(const RouteBwdLaunch& r, hipStream_t st) {
  if (r.act_bf16) route_bwd_t<bf16_t>(r, st);
  else route_bwd_t<float>(r, st);
}

}  // namespace moe

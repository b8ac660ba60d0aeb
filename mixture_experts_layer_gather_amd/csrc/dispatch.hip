// Dispatch and combine kernels (gfx950): the token permutation into
// expert-contiguous rows and its inverse, forward and backward.
//
// Dispatch sends each token to its experts following the routing map and
// combine returns the expert outputs to token order with high-precision
// accumulation (Hybrid-EP article, paragraphs on the dispatch/combine
// operators, the routing map and hierarchical accumulation). On one GPU the
// transfer becomes a gather into an HBM buffer: each token row is read once
// and written k times with 16-byte stores; combine is a per-token gather in
// fp32, in slot order, with no atomics (deterministic).
//
// Row order: expert ascending, then token ascending. Ranks inside a chunk of
// tokens come from per-expert token bitmasks in LDS (popcount of the lower
// bits), never from the order in which atomics land.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

int64_t dispatch_chunks(int64_t T) { return (T + kChunkTok - 1) / kChunkTok; }

// --- 1. per-chunk expert histogram --------------------------------------
__global__ __launch_bounds__(256) void dispatch_count_kernel(const int32_t* __restrict__ idx,
                                                             int32_t* __restrict__ chunk_cnt,
                                                             int T, int E, int k) {
  extern __shared__ int32_t hist[];
  const int c = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += 256) hist[e] = 0;
  __syncthreads();
  const int t = c * kChunkTok + threadIdx.x;
  if (t < T)
    for (int j = 0; j < k; ++j) atomicAdd(&hist[idx[int64_t(t) * k + j]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) chunk_cnt[int64_t(c) * E + e] = hist[e];
}

// --- 2. scan over (chunk, expert) -----------------------------------------
// chunk_cnt[c][e] becomes the first row of expert e's tokens in chunk c.
// Thread e owns expert e: its column is read twice with 16 loads in flight
// (totals, then running bases); the exclusive scan of the totals over the
// experts runs on wave shuffles. Integer sums: the order does not matter.
__global__ __launch_bounds__(1024) void dispatch_scan_kernel(int32_t* __restrict__ chunk_cnt,
                                                             int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ offsets,
                                                             int nchunks, int E) {
  constexpr int B = 16;
  __shared__ int32_t s_wave[16];
  const int e = threadIdx.x;
  const int lane = lane_id(), wave = e / kWave;
  int32_t total = 0;
  if (e < E) {
    for (int c0 = 0; c0 < nchunks; c0 += B) {
      int32_t v[B];
#pragma unroll
      for (int j = 0; j < B; ++j) v[j] = (c0 + j < nchunks) ? chunk_cnt[int64_t(c0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < B; ++j) total += v[j];
    }
  }
  // inclusive scan of the totals within each wave, then across waves
  int32_t inc = total;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int32_t u = __shfl_up(inc, o, kWave);
    if (lane >= o) inc += u;
  }
  if (lane == kWave - 1) s_wave[wave] = inc;
  __syncthreads();
  int32_t before = 0;
  for (int w = 0; w < wave; ++w) before += s_wave[w];
  const int32_t base = before + inc - total;  // exclusive prefix over experts
  if (e < E) {
    int32_t run = base;
    for (int c0 = 0; c0 < nchunks; c0 += B) {
      int32_t v[B];
#pragma unroll
      for (int j = 0; j < B; ++j) v[j] = (c0 + j < nchunks) ? chunk_cnt[int64_t(c0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < B; ++j) {
        if (c0 + j < nchunks) chunk_cnt[int64_t(c0 + j) * E + e] = run;
        run += v[j];
      }
    }
    counts[e] = total;
    offsets[e] = base;
    if (e == E - 1) offsets[E] = base + total;
  }
}

// --- 3. positions: row of every (token, slot) -----------------------------
// SCAN = false: chunk_base holds the scanned bases (kernel 2).
// SCAN = true (few chunks): chunk_base holds the raw per-chunk counts of
// kernel 1, and every block derives its own chunk's bases from them (expert
// totals, their exclusive scan, plus the earlier chunks' counts; integer sums
// in any order); block 0 also writes counts and offsets. One launch fewer.
// SCAN = true up to this many chunks (measured: 16 chunks x 8 experts 8.9 ->
// 6.1 us for scan + positions; 64 chunks x 128 experts 14.0 -> 14.9 us)
constexpr int kScanInPosChunks = 32;
template <bool SCAN>
__global__ __launch_bounds__(256) void dispatch_pos_kernel(const int32_t* __restrict__ idx,
                                                           const int32_t* __restrict__ chunk_base,
                                                           int32_t* __restrict__ counts,
                                                           int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ row_id_map,
                                                           int32_t* __restrict__ perm_token,
                                                           int T, int E, int k) {
  // bits[e][w]: bit b set when token c*256 + 32w + b of this chunk goes to e;
  // SCAN: s_base[e] = first row of expert e's tokens in this chunk
  extern __shared__ uint32_t bits[];
  constexpr int W = kChunkTok / 32;
  const int c = blockIdx.x;
  int32_t* s_base = reinterpret_cast<int32_t*>(bits + E * W);
  for (int i = threadIdx.x; i < E * W; i += 256) bits[i] = 0;
  if constexpr (SCAN) {
    __shared__ int32_t s_wave[4];
    const int nchunks = (T + kChunkTok - 1) / kChunkTok;
    // thread t owns experts 4t .. 4t + 3 (E <= 1024)
    int32_t tot[4] = {0, 0, 0, 0}, pre[4] = {0, 0, 0, 0};
    const int e0 = 4 * threadIdx.x;
    if (e0 < E) {
      // 8 chunks' loads in flight at a time; 16-byte loads when rows allow
      const bool vec = (E & 3) == 0;
      for (int c0 = 0; c0 < nchunks; c0 += 8) {
        int4 v[8];
#pragma unroll
        for (int b = 0; b < 8; ++b) {
          const int cc = c0 + b;
          const int32_t* p = chunk_base + int64_t(cc) * E + e0;
          if (cc >= nchunks) v[b] = make_int4(0, 0, 0, 0);
          else if (vec) v[b] = *reinterpret_cast<const int4*>(p);
          else v[b] = make_int4(p[0], e0 + 1 < E ? p[1] : 0, e0 + 2 < E ? p[2] : 0, e0 + 3 < E ? p[3] : 0);
        }
#pragma unroll
        for (int b = 0; b < 8; ++b) {
          const int32_t w4[4] = {v[b].x, v[b].y, v[b].z, v[b].w};
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            tot[u] += w4[u];
            if (c0 + b < c) pre[u] += w4[u];
          }
        }
      }
    }
    const int32_t mine = tot[0] + tot[1] + tot[2] + tot[3];
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    int32_t inc = mine;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int32_t u = __shfl_up(inc, o, kWave);
      if (lane >= o) inc += u;
    }
    if (lane == kWave - 1) s_wave[wave] = inc;
    __syncthreads();
    int32_t before = 0;
    for (int w = 0; w < wave; ++w) before += s_wave[w];
    int32_t run = before + inc - mine;  // exclusive prefix over experts < e0
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = e0 + u;
      if (e < E) {
        s_base[e] = run + pre[u];
        if (c == 0) {
          counts[e] = tot[u];
          offsets[e] = run;
          if (e == E - 1) offsets[E] = run + tot[u];
        }
      }
      run += tot[u];
    }
  }
  __syncthreads();
  const int tl = threadIdx.x;
  const int t = c * kChunkTok + tl;
  int32_t my[16];
  if (t < T) {
    _Pragma("unroll") for (int j = 0; j < 16; ++j) if (j < k) {
      my[j] = idx[int64_t(t) * k + j];
      atomicOr(&bits[my[j] * W + (tl >> 5)], 1u << (tl & 31));
    }
  }
  __syncthreads();
  if (t < T) {
    const int w = tl >> 5;
    const uint32_t below = (1u << (tl & 31)) - 1u;
    _Pragma("unroll") for (int j = 0; j < 16; ++j) if (j < k) {
      const int e = my[j];
      const uint32_t* be = bits + e * W;
      int rank = __popc(be[w] & below);
      for (int i = 0; i < w; ++i) rank += __popc(be[i]);
      const int32_t row = (SCAN ? s_base[e] : chunk_base[int64_t(c) * E + e]) + rank;
      row_id_map[int64_t(t) * k + j] = row;
      perm_token[row] = t;
    }
  }
}

// --- 4. gather: x_perm[row_id_map[t,j]] = x[t] -----------------------------
// One group of G = d/VEC threads per token, 16 bytes per thread per step.
template <typename T>
__global__ __launch_bounds__(256) void dispatch_gather_kernel(const T* __restrict__ x,
                                                              const int32_t* __restrict__ row_id_map,
                                                              T* __restrict__ x_perm, int ntok,
                                                              int d, int k, int tpb) {
  constexpr int VEC = 16 / sizeof(T);
  const int chunks = d / VEC;
  const int per = 256 / tpb;  // threads per token
  const int sub = threadIdx.x / per;
  const int t = blockIdx.x * tpb + sub;
  if (t >= ntok || sub >= tpb) return;
  int32_t rows[16];
  _Pragma("unroll") for (int j = 0; j < 16; ++j) if (j < k) rows[j] = row_id_map[int64_t(t) * k + j];
  const uint4* src = reinterpret_cast<const uint4*>(x + int64_t(t) * d);
  for (int ch = threadIdx.x % per; ch < chunks; ch += per) {
    const uint4 v = src[ch];
    _Pragma("unroll") for (int j = 0; j < 16; ++j) if (j < k)
      reinterpret_cast<uint4*>(x_perm + int64_t(rows[j]) * d)[ch] = v;
  }
}

// FP8 variant: each token is quantised once per 1 x 128 block (scale =
// amax / 448, fp32 divide; 1 for an all-zero block; E4M3 round to nearest
// even via v_cvt_pk_fp8_f32) and its codes and scales are written k times.
// 16 lanes cover one 128-element block (8 bf16 per lane).
__global__ __launch_bounds__(256) void dispatch_gather_fp8_kernel(
    const bf16_t* __restrict__ x, const int32_t* __restrict__ row_id_map,
    uint8_t* __restrict__ xq, float* __restrict__ xs, int ntok, int d, int k) {
  const int t = blockIdx.x;
  if (t >= ntok) return;
  int32_t rows[16];
  _Pragma("unroll") for (int j = 0; j < 16; ++j) if (j < k) rows[j] = row_id_map[int64_t(t) * k + j];
  const int nblk = d / 128;
  const int chunks = d / 8;
  // all threads of the block iterate the same number of times so that the
  // 16-lane shuffles always see full groups
  for (int base = 0; base < chunks; base += 256) {
    const int ch = base + threadIdx.x;
    const bool ok = ch < chunks;
    float v[8];
    if (ok) Vec16<bf16_t>::load(x + int64_t(t) * d + int64_t(ch) * 8, v);
    else
      for (int i = 0; i < 8; ++i) v[i] = 0.0f;
    float amax = 0.0f;
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    for (int o = 8; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, kWave));
    const float scale = (amax == 0.0f) ? 1.0f : amax / 448.0f;
    const u32x2 w = fp8_encode8(v, scale, 1.0f / scale, fp8_fast_scale(scale));
    const uint32_t lo = w[0], hi = w[1];
    if (ok) {
      const int blk = ch / 16;
      _Pragma("unroll") for (int j = 0; j < 16; ++j) if (j < k) {
        *reinterpret_cast<uint2*>(xq + int64_t(rows[j]) * d + int64_t(ch) * 8) = make_uint2(lo, hi);
        if ((ch & 15) == 0) xs[int64_t(rows[j]) * nblk + blk] = scale;
      }
    }
  }
}

// MXFP8 variant: 1 x 32 blocks, 4 lanes per block; codes of x * 2^-e with
// the E8M0 byte e + 127 per block (e from mx_scale_exp, as in the MXFP8
// quantiser of the expert GEMMs), written k times.
__global__ __launch_bounds__(256) void dispatch_gather_mx_kernel(
    const bf16_t* __restrict__ x, const int32_t* __restrict__ row_id_map,
    uint8_t* __restrict__ xq, uint8_t* __restrict__ xs, int ntok, int d, int k) {
  const int t = blockIdx.x;
  if (t >= ntok) return;
  int32_t rows[16];
  _Pragma("unroll") for (int j = 0; j < 16; ++j) if (j < k) rows[j] = row_id_map[int64_t(t) * k + j];
  const int nblk = d / 32;
  const int chunks = d / 8;
  for (int base = 0; base < chunks; base += 256) {
    const int ch = base + threadIdx.x;
    const bool ok = ch < chunks;
    float v[8];
    if (ok) Vec16<bf16_t>::load(x + int64_t(t) * d + int64_t(ch) * 8, v);
    else
      for (int i = 0; i < 8; ++i) v[i] = 0.0f;
    float amax = 0.0f;
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    for (int o = 2; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, kWave));
    const int e = mx_scale_exp(amax);
    const u32x2 c = mx_codes8(v, e);
    if (ok) {
      _Pragma("unroll") for (int j = 0; j < 16; ++j) if (j < k) {
        *reinterpret_cast<uint2*>(xq + int64_t(rows[j]) * d + int64_t(ch) * 8) = make_uint2(c[0], c[1]);
        if ((ch & 3) == 0) xs[int64_t(rows[j]) * nblk + ch / 4] = uint8_t(e + 127);
      }
    }
  }
}

static int tokens_per_block(int64_t d, int vec) {
  const int64_t per = d / vec;
  if (per >= 256) return 1;
  int tpb = 1;
  while (tpb * 2 * per <= 256) tpb *= 2;
  return tpb;
}

void launch_dispatch(const DispatchLaunch& a, hipStream_t st) {
  const int T = int(a.T), E = int(a.E), k = int(a.k);
  const int nchunks = int(dispatch_chunks(a.T));
  if (!a.counted)
    dispatch_count_kernel<<<nchunks, 256, sizeof(int32_t) * E, st>>>(a.idx, a.chunk_base, T, E, k);
  const size_t bits_lds = sizeof(uint32_t) * E * (kChunkTok / 32);
  if (nchunks <= kScanInPosChunks) {
    dispatch_pos_kernel<true><<<nchunks, 256, bits_lds + sizeof(int32_t) * E, st>>>(
        a.idx, a.chunk_base, a.counts, a.offsets, a.row_id_map, a.perm_token, T, E, k);
  } else {
    dispatch_scan_kernel<<<1, 1024, 0, st>>>(a.chunk_base, a.counts, a.offsets, nchunks, E);
    dispatch_pos_kernel<false><<<nchunks, 256, bits_lds, st>>>(a.idx, a.chunk_base, a.counts, a.offsets,
                                                               a.row_id_map, a.perm_token, T, E, k);
  }
  if (a.mx) {
    dispatch_gather_mx_kernel<<<T, 256, 0, st>>>(reinterpret_cast<const bf16_t*>(a.x), a.row_id_map,
                                                 reinterpret_cast<uint8_t*>(a.x_perm),
                                                 reinterpret_cast<uint8_t*>(a.x_scale), T, int(a.d), k);
  } else if (a.fp8) {
    dispatch_gather_fp8_kernel<<<T, 256, 0, st>>>(reinterpret_cast<const bf16_t*>(a.x), a.row_id_map,
                                                  reinterpret_cast<uint8_t*>(a.x_perm), a.x_scale, T,
                                                  int(a.d), k);
  } else if (a.act == 1) {
    const int tpb = tokens_per_block(a.d, 8);
    dispatch_gather_kernel<bf16_t><<<(T + tpb - 1) / tpb, 256, 0, st>>>(
        reinterpret_cast<const bf16_t*>(a.x), a.row_id_map, reinterpret_cast<bf16_t*>(a.x_perm), T,
        int(a.d), k, tpb);
  } else {
    const int tpb = tokens_per_block(a.d, 4);
    dispatch_gather_kernel<float><<<(T + tpb - 1) / tpb, 256, 0, st>>>(
        reinterpret_cast<const float*>(a.x), a.row_id_map, reinterpret_cast<float*>(a.x_perm), T,
        int(a.d), k, tpb);
  }
}

// --- combine / dispatch backward: per-token ordered gather ----------------
// dst[t] = sum_j g[t,j] * src[row_id_map[t,j]] (+ add[t]), fp32 in slot
// order, the added term last, one rounding.
template <typename T, int KMAX>
__global__ __launch_bounds__(256) void combine_kernel(const T* __restrict__ src,
                                                      const int32_t* __restrict__ row_id_map,
                                                      const float* __restrict__ gate,
                                                      const T* __restrict__ add, T* __restrict__ dst,
                                                      int ntok, int d, int k, int tpb) {
  constexpr int VEC = 16 / sizeof(T);
  // chunks per pass: every load of a pass is issued before any arithmetic,
  // so a thread keeps NC (k + 1) 16-byte loads in flight
  constexpr int NC = KMAX <= 4 ? 2 : 1;
  const int chunks = d / VEC;
  const int per = 256 / tpb;
  const int sub = threadIdx.x / per;
  const int t = blockIdx.x * tpb + sub;
  if (t >= ntok || sub >= tpb) return;
  int32_t rows[KMAX];
  float g[KMAX];
  _Pragma("unroll") for (int j = 0; j < KMAX; ++j) if (j < k) {
    rows[j] = row_id_map[int64_t(t) * k + j];
    g[j] = gate ? gate[int64_t(t) * k + j] : 1.0f;
  }
  for (int ch0 = threadIdx.x % per; ch0 < chunks; ch0 += NC * per) {
    uint4 raw[NC][KMAX + 1];
    _Pragma("unroll") for (int h = 0; h < NC; ++h) {
      const int ch = ch0 + h * per;
      if (ch < chunks) {
        _Pragma("unroll") for (int j = 0; j < KMAX; ++j) if (j < k)
          raw[h][j] = ld_stream(src + int64_t(rows[j]) * d + int64_t(ch) * VEC);
        if (add) raw[h][KMAX] = ld_stream(add + int64_t(t) * d + int64_t(ch) * VEC);
      }
    }
    _Pragma("unroll") for (int h = 0; h < NC; ++h) {
      const int ch = ch0 + h * per;
      if (ch >= chunks) break;
      float acc[VEC];
      for (int i = 0; i < VEC; ++i) acc[i] = 0.0f;
      _Pragma("unroll") for (int j = 0; j < KMAX; ++j) if (j < k) {
        float v[VEC];
        Vec16<T>::unpack(raw[h][j], v);
        for (int i = 0; i < VEC; ++i) acc[i] = __builtin_fmaf(g[j], v[i], acc[i]);
      }
      if (add) {
        float v[VEC];
        Vec16<T>::unpack(raw[h][KMAX], v);
        for (int i = 0; i < VEC; ++i) acc[i] += v[i];
      }
      st_stream(dst + int64_t(t) * d + int64_t(ch) * VEC, Vec16<T>::pack(acc));
    }
  }
}

template <typename T, int KMAX>
static void combine_t(const CombineLaunch& a, int tpb, hipStream_t st) {
  combine_kernel<T, KMAX><<<(a.T + tpb - 1) / tpb, 256, 0, st>>>(
      reinterpret_cast<const T*>(a.src), a.row_id_map, a.gate, reinterpret_cast<const T*>(a.add),
      reinterpret_cast<T*>(a.dst), int(a.T), int(a.d), int(a.k), tpb);
}
template <typename T>
static void combine_k(const CombineLaunch& a, hipStream_t st) {
  const int tpb = tokens_per_block(a.d, 16 / int(sizeof(T)));
  if (a.k <= 2) combine_t<T, 2>(a, tpb, st);
  else if (a.k <= 4) combine_t<T, 4>(a, tpb, st);
  else if (a.k <= 8) combine_t<T, 8>(a, tpb, st);
  else combine_t<T, 16>(a, tpb, st);
}

void launch_combine(const CombineLaunch& a, hipStream_t st) {
  if (a.act == 1) combine_k<bf16_t>(a, st);
  else combine_k<float>(a, st);
}

// --- combine backward: one block per token --------------------------------
template <typename T, int KMAX>
__global__ __launch_bounds__(256) void combine_bwd_kernel(const T* __restrict__ dy,
                                                          const T* __restrict__ out_perm,
                                                          const int32_t* __restrict__ row_id_map,
                                                          const float* __restrict__ gate,
                                                          T* __restrict__ d_out, float* __restrict__ d_gate,
                                                          int d, int k) {
  constexpr int VEC = 16 / sizeof(T);
  __shared__ float red[4][16];
  const int t = blockIdx.x;
  const int chunks = d / VEC;
  int32_t rows[KMAX];
  float g[KMAX], part[KMAX];
  for (int j = 0; j < KMAX; ++j) part[j] = 0.0f;
  _Pragma("unroll") for (int j = 0; j < KMAX; ++j) if (j < k) {
    rows[j] = row_id_map[int64_t(t) * k + j];
    g[j] = gate[int64_t(t) * k + j];
  }
  for (int ch = threadIdx.x; ch < chunks; ch += 256) {
    float dv[VEC];
    Vec16<T>::unpack(ld_stream(dy + int64_t(t) * d + int64_t(ch) * VEC), dv);
    uint4 raw[KMAX];
    _Pragma("unroll") for (int j = 0; j < KMAX; ++j) if (j < k)
      raw[j] = ld_stream(out_perm + int64_t(rows[j]) * d + int64_t(ch) * VEC);
    _Pragma("unroll") for (int j = 0; j < KMAX; ++j) if (j < k) {
      float o[VEC], w[VEC];
      Vec16<T>::unpack(raw[j], o);
      float s = 0.0f;
      for (int i = 0; i < VEC; ++i) {
        s = __builtin_fmaf(dv[i], o[i], s);
        w[i] = g[j] * dv[i];
      }
      part[j] += s;
      st_stream(d_out + int64_t(rows[j]) * d + int64_t(ch) * VEC, Vec16<T>::pack(w));
    }
  }
  const int wave = threadIdx.x / kWave;
  _Pragma("unroll") for (int j = 0; j < KMAX; ++j) if (j < k) {
    const float s = wave_sum(part[j]);
    if (lane_id() == 0) red[wave][j] = s;
  }
  __syncthreads();
  if (threadIdx.x < k) {
    const int j = threadIdx.x;
    d_gate[int64_t(t) * k + j] = ((red[0][j] + red[1][j]) + red[2][j]) + red[3][j];
  }
}

template <typename T, int KMAX>
static void combine_bwd_t(const CombineBwdLaunch& a, hipStream_t st) {
  combine_bwd_kernel<T, KMAX><<<a.T, 256, 0, st>>>(
      reinterpret_cast<const T*>(a.dy), reinterpret_cast<const T*>(a.out_perm), a.row_id_map, a.gate,
      reinterpret_cast<T*>(a.d_out_perm), a.d_gate, int(a.d), int(a.k));
}
template <typename T>
static void combine_bwd_k(const CombineBwdLaunch& a, hipStream_t st) {
  if (a.k <= 2) combine_bwd_t<T, 2>(a, st);
  else if (a.k <= 4) combine_bwd_t<T, 4>(a, st);
  else if (a.k <= 8) combine_bwd_t<T, 8>(a, st);
  else combine_bwd_t<T, 16>(a, st);
}

void launch_combine_bwd(const CombineBwdLaunch& a, hipStream_t st) {
  if (a.act == 1) combine_bwd_k<bf16_t>(a, st);
  else combine_bwd_k<float>(a, st);
}

// --- FP8 block quantisation (weights 128x128, activations 1x128) ---------
// One workgroup per block: amax by a fixed-order reduction, then codes.
template <typename T>
__global__ __launch_bounds__(256) void quant_blocks_kernel(const T* __restrict__ src, uint8_t* __restrict__ dst,
                                                           float* __restrict__ scale, int64_t rows,
                                                           int64_t cols, int br, int bc, int nbc) {
  __shared__ float red[4];
  const int64_t I = blockIdx.y, J = blockIdx.x;
  const int64_t r0 = I * br, c0 = J * bc;
  const int64_t r1 = min<int64_t>(r0 + br, rows), c1 = min<int64_t>(c0 + bc, cols);
  const int w = int(c1 - c0);
  const int n = int(r1 - r0) * w;
  float amax = 0.0f;
  for (int i = threadIdx.x; i < n; i += 256) {
    const int64_t r = r0 + i / w, c = c0 + i % w;
    amax = fmaxf(amax, fabsf(Elem<T>::load(src + r * cols + c)));
  }
  amax = wave_max(amax);
  if (lane_id() == 0) red[threadIdx.x / kWave] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = (amax == 0.0f) ? 1.0f : amax / 448.0f;
  if (threadIdx.x == 0) scale[I * nbc + J] = s;
  for (int i = threadIdx.x; i < n; i += 256) {
    const int64_t r = r0 + i / w, c = c0 + i % w;
    const float v = Elem<T>::load(src + r * cols + c) / s;
    dst[r * cols + c] = uint8_t(__builtin_amdgcn_cvt_pk_fp8_f32(v, 0.0f, 0, false) & 0xff);
  }
}

// Whole 128 x 128 blocks (the weight layout): the block stays in registers
// between the amax and the codes, so the source is read once. Thread t holds
// columns 8 (t % 16) .. + 8 of rows t / 16 + 16 i (i < 8): 16-byte loads, a
// group of 16 threads covers one 256- (bf16) or 512-byte (fp32) row segment;
// the codes leave as 8-byte stores. Same scale and per-element arithmetic as
// quant_blocks_kernel.
template <typename T>
__global__ __launch_bounds__(256) void quant_tiles128_kernel(const T* __restrict__ src, uint8_t* __restrict__ dst,
                                                             float* __restrict__ scale, int64_t cols, int nbc) {
  __shared__ float red[4];
  const int64_t I = blockIdx.y, J = blockIdx.x;
  const int c = int(threadIdx.x % 16) * 8, rw = int(threadIdx.x / 16);
  const int64_t base = (I * 128 + rw) * cols + J * 128 + c;
  float v[8][8];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const T* p = src + base + int64_t(16 * i) * cols;
    if constexpr (sizeof(T) == 2) {
      Vec16<bf16_t>::load(p, v[i]);
    } else {
      Vec16<float>::load(p, v[i]);
      Vec16<float>::load(p + 4, v[i] + 4);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[i][e]));
  }
  amax = wave_max(amax);
  if (lane_id() == 0) red[threadIdx.x / kWave] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = (amax == 0.0f) ? 1.0f : amax / 448.0f;
  if (threadIdx.x == 0) scale[I * nbc + J] = s;
  const float r = 1.0f / s;
  const bool fast = fp8_fast_scale(s);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const u32x2 w = fp8_encode8(v[i], s, r, fast);
    *reinterpret_cast<uint2*>(dst + base + int64_t(16 * i) * cols) = make_uint2(w[0], w[1]);
  }
}

void launch_quant_blocks(const QuantLaunch& a, hipStream_t st) {
  const int nbr = int((a.rows + a.br - 1) / a.br), nbc = int((a.cols + a.bc - 1) / a.bc);
  const dim3 grid(nbc, nbr);
  const bool tiles = a.br == 128 && a.bc == 128 && a.rows % 128 == 0 && a.cols % 128 == 0 &&
                     (reinterpret_cast<uintptr_t>(a.src) & 15) == 0 && (reinterpret_cast<uintptr_t>(a.dst) & 15) == 0;
  if (tiles) {
    if (a.src_bf16)
      quant_tiles128_kernel<bf16_t><<<grid, 256, 0, st>>>(reinterpret_cast<const bf16_t*>(a.src), a.dst, a.scale,
                                                          a.cols, nbc);
    else
      quant_tiles128_kernel<float><<<grid, 256, 0, st>>>(reinterpret_cast<const float*>(a.src), a.dst, a.scale,
                                                         a.cols, nbc);
  } else if (a.src_bf16)
    quant_blocks_kernel<bf16_t><<<grid, 256, 0, st>>>(reinterpret_cast<const bf16_t*>(a.src), a.dst,
                                                      a.scale, a.rows, a.cols, int(a.br), int(a.bc), nbc);
  else
    quant_blocks_kernel<float><<<grid, 256, 0, st>>>(reinterpret_cast<const float*>(a.src), a.dst,
                                                     a.scale, a.rows, a.cols, int(a.br), int(a.bc), nbc);
}

}  // namespace moe

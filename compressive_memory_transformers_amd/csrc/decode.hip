// Streaming decode: one new token per (batch, head) on top of the carried
// state and the current segment's key/value cache.
//
// "Infini-Attention" (AI Wiki), "Why is the memory footprint bounded?": a
// stream runs segment by segment with only (M, z) carried, so a token's work
// is bounded by the segment length. For the token at position pos of its
// segment: local causal attention over the segment's rows 0..pos, retrieval
// A_mem = sigma(q) M / (sigma(q) z) from the state before the segment, the
// sigmoid(beta) gate ("What happens inside the Infini-attention block?").
//
// Two kernels, memory-bound (the cache is read once per step):
//   partial: per (batch, KV head, chunk of 64 cache rows), the grouped query
//            heads' scores, the chunk maximum and exp2 weight sum, and the
//            weighted value sums; the workgroup whose chunk holds row pos also
//            appends the token's key and value to the cache (no workgroup
//            reads that row from the cache in this step: it takes the new
//            key/value directly);
//   combine: per (batch, KV head, 32 output columns), the chunks merged by
//            their maxima, the retrieval from the float state, the gate.
// The fold of a full segment into (M, z) reuses the recurrence kernels
// (api.hip).
#include "common.hpp"
#include "kernels.hpp"
#include "lds_tile.hpp"

namespace infini {

namespace {

constexpr int kDecodeKC = 64;   // cache rows per partial workgroup (one wave)
constexpr int kDecodeNT = 256;  // threads per combine workgroup

template <typename T, int W>
__device__ __forceinline__ const T* cache_row(const DecodeArgs& a, const T* cache, const T* fresh,
                                              int t) {
  return t == a.pos ? fresh : cache + (int64_t)t * W;
}

// One 256-thread workgroup per (batch, KV head, chunk of 64 cache rows).
// Thread (row r = tid / 4, quarter u = tid % 4) loads columns [u d/4,
// (u+1) d/4) of row r of K and of V at once (one memory latency for the whole chunk); the
// four quarters' partial scores are summed by DPP; one wave per head takes the
// chunk maximum and weight sum; the value sums run over (head, 8-column group,
// quarter of the rows) triples and are added in LDS.
// DK: the key width (q, k, rows of M); DV: the value width (v, the output).
// GM: the largest group the instantiation serves (its LDS is sized for it).
template <typename T, int DK, int DV, int GM>
__global__ __launch_bounds__(256) void decode_partial_kernel(DecodeArgs a) {
  constexpr int KC = kDecodeKC, C8 = DV / 8;
  static_assert(GM <= kDecodeMaxGroup, "group bucket");
  // columns and 8-column chunks of a row quarter, of K and of V
  constexpr int QWK = DK / 4, QCK = QWK / 8, QWV = DV / 4, QCV = QWV / 8;
  __shared__ float qs[GM * DK];  // the group's queries, scaled by log2(e) / sqrt(d_key)
  __shared__ float ps[GM * KC];  // scores, then exp2 weights
  __shared__ __align__(16) T vs[KC * DV];
  __shared__ float ov[4 * GM * DV];  // value sums of the four row quarters

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int G = a.G;
  const int n_part = a.B * a.Hkv * a.n_chunks;
  if ((int)blockIdx.x >= n_part) {
    // the retrieval workgroups, one per (batch, KV head, 32-column slab):
    // numerator sigma(q) M[:, slab] and denominator sigma(q) . z of the
    // group's heads, from the state before the segment (the combine reads
    // them after this launch)
    const int rb = (int)blockIdx.x - n_part;
    const int ru = rb / (DV / 32), slab = rb % (DV / 32);
    const int b = ru / a.Hkv, j = ru % a.Hkv;
    const T* q = static_cast<const T*>(a.q) + ((int64_t)b * a.Hq + (int64_t)j * G) * DK;
    const float* M = a.M + (int64_t)ru * DK * DV + 32 * slab;
    const float* z = a.z + (int64_t)ru * DK;
    float* sq = qs;  // sigma(q) of the group, [G][DK]
    for (int x = tid; x < G * DK; x += 256) sq[x] = feature_map(to_f32<T>(q[x]));
    __syncthreads();
    if (slab == 0) {  // per head (32 lanes a head): den
      for (int g0 = 0; g0 < G; g0 += 8) {
        const int g = g0 + tid / 32, l32 = tid & 31;
        if (g < G) {
          float dp = 0.f;
          for (int k = l32; k < DK; k += 32) dp += sq[g * DK + k] * z[k];
#pragma unroll
          for (int o = 16; o > 0; o >>= 1) dp += __shfl_xor(dp, o, 32);
          if (l32 == 0) a.rden[ru * G + g] = dp;
        }
      }
    }
    for (int x = tid; x < G * 32; x += 256) {
      const int g = x / 32, cs = x % 32;
      float r = 0.f;
#pragma unroll 16
      for (int k = 0; k < DK; ++k) r += sq[g * DK + k] * M[(int64_t)k * DV + cs];
      a.retr[((int64_t)ru * G + g) * DV + 32 * slab + cs] = r;
    }
    return;
  }
  const int unit = blockIdx.x / a.n_chunks, ch = blockIdx.x % a.n_chunks;
  const int b = unit / a.Hkv, j = unit % a.Hkv;
  const int t0 = ch * KC;
  const int n = min(KC, a.pos + 1 - t0);  // rows of this chunk, >= 1
  const T* q = static_cast<const T*>(a.q) + ((int64_t)b * a.Hq + (int64_t)j * G) * DK;
  const T* knew = static_cast<const T*>(a.k) + (int64_t)unit * DK;
  const T* vnew = static_cast<const T*>(a.v) + (int64_t)unit * DV;
  const T* kc = static_cast<const T*>(a.k_cache) + (int64_t)unit * a.seg_len * DK;
  const T* vc = static_cast<const T*>(a.v_cache) + (int64_t)unit * a.seg_len * DV;

  // this thread's quarter row (a row past the chunk repeats row t0: finite, weight 0)
  const int r = tid >> 2, u = tid & 3;
  const int t = t0 + (r < n ? r : 0);
  const T* krow = cache_row<T, DK>(a, kc, knew, t) + QWK * u;
  const T* vrow = cache_row<T, DV>(a, vc, vnew, t) + QWV * u;
  frag_t<T> kv[QCK], vv[QCV];
#pragma unroll
  for (int c = 0; c < QCK; ++c) kv[c] = load8<T>(krow + 8 * c);
#pragma unroll
  for (int c = 0; c < QCV; ++c) vv[c] = load8<T>(vrow + 8 * c);
  for (int x = tid; x < G * DK; x += 256) qs[x] = to_f32<T>(q[x]) * a.scale_log2;
#pragma unroll
  for (int c = 0; c < QCV; ++c) store8<T>(vs + r * DV + QWV * u + 8 * c, vv[c]);
  __syncthreads();

  // scores: the quarter's partial dot for every head, summed over the quad
  for (int g = 0; g < G; ++g) {
      float sp = 0.f;
#pragma unroll
      for (int c = 0; c < QCK; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) sp += to_f32<T>(kv[c][e]) * qs[g * DK + QWK * u + 8 * c + e];
      sp = row_sum<4>(sp);
      if (u == 0) ps[g * KC + r] = r < n ? sp : -INFINITY;
    }
  __syncthreads();

  // per head (one wave a head): chunk maximum and weight sum, lane = row
  float* part = a.part + ((int64_t)unit * a.n_chunks + ch) * G * (DV + 2);
  for (int g = w; g < G; g += 4) {
    const float sc = ps[g * KC + lane];
    const float m = wave_max(sc);
    const float p = exp2f(sc - m);  // 0 past the chunk's rows
    const float l = wave_sum(p);
    ps[g * KC + lane] = p;
    if (lane == 0) {
      part[g * (DV + 2)] = m;
      part[g * (DV + 2) + 1] = l;
    }
  }
  __syncthreads();

  // value sums: (head, 8-column group, row quarter) triples
  for (int x = tid; x < G * C8 * 4; x += 256) {
    const int kq = x / (G * C8), pr = x % (G * C8);
    const int g = pr / C8, c = pr % C8;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll 4
    for (int i = 0; i < KC / 4; ++i) {
      const int tt = kq * (KC / 4) + i;  // rows past n carry weight 0
      const frag_t<T> vx = load8<T>(vs + tt * DV + 8 * c);
      const float wgt = ps[g * KC + tt];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += wgt * to_f32<T>(vx[e]);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) ov[(kq * G + g) * DV + 8 * c + e] = acc[e];
  }
  __syncthreads();
  for (int x = tid; x < G * DV; x += 256) {
    const int g = x / DV, col = x % DV;
    part[g * (DV + 2) + 2 + col] = (ov[(0 * G + g) * DV + col] + ov[(1 * G + g) * DV + col]) +
                                   (ov[(2 * G + g) * DV + col] + ov[(3 * G + g) * DV + col]);
  }

  // append the token to the cache (no workgroup reads row pos from the cache)
  if (t0 <= a.pos && a.pos < t0 + KC) {
    T* kw = static_cast<T*>(a.k_cache) + ((int64_t)unit * a.seg_len + a.pos) * DK;
    T* vw = static_cast<T*>(a.v_cache) + ((int64_t)unit * a.seg_len + a.pos) * DV;
    for (int x = tid; x < DK; x += 256) kw[x] = knew[x];
    for (int x = tid; x < DV; x += 256) vw[x] = vnew[x];
  }
}

// Per (batch, KV head, 32-column slab of the output): merge the chunks by
// their maxima, add the retrieval the partial launch formed, gate. The
// chunks' maxima, weight sums and value sums are loaded at once into LDS;
// the small reductions run across the workgroup.
template <typename T, int DK, int DV>
__global__ __launch_bounds__(kDecodeNT) void decode_combine_kernel(DecodeArgs a) {
  constexpr int NT = kDecodeNT, GM = kDecodeMaxGroup, NCM = kDecodeMaxChunks;
  __shared__ float wch[GM * NCM]; // chunk maxima, then weights exp2(m_c - m)
  __shared__ float lch[GM * NCM]; // chunk weight sums
  __shared__ float gate[GM], lsum[GM];
  constexpr int OC = 4096;           // staged value sums: chunks x heads x 32 columns
  __shared__ float os[OC];

  const int tid = threadIdx.x;
  const int G = a.G, NC = a.n_chunks;
  const int unit = blockIdx.x / (DV / 32), slab = blockIdx.x % (DV / 32);
  const int b = unit / a.Hkv, j = unit % a.Hkv;
  const int hq0 = j * G;
  const float* part = a.part + (int64_t)unit * NC * G * (DV + 2);

  for (int x = tid; x < G * NC; x += NT) {  // chunk maxima and weight sums
    const float* pc = part + ((x % NC) * G + x / NC) * (DV + 2);
    wch[(x / NC) * NCM + x % NC] = pc[0];
    lch[(x / NC) * NCM + x % NC] = pc[1];
  }
  // the slab's value sums of every (chunk, head), when they fit (G * NC <= 128)
  const bool staged = G * NC * 32 <= OC;
  if (staged)
    for (int x = tid; x < G * NC * 8; x += NT) {  // 8 float4 per (chunk, head)
      const int cg = x / 8, c4 = x % 8;
      const float* src = part + cg * (DV + 2) + 2 + 32 * slab + 4 * c4;
      f32x4 y;
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = src[e];  // rows of D + 2 floats: 8-byte aligned only
      *reinterpret_cast<f32x4*>(os + cg * 32 + 4 * c4) = y;
    }
  __syncthreads();
  // per head (32 lanes a head): the chunks' maximum m (every lane gets it
  // from the butterfly), the weights exp2(m_c - m) and the weight sum
  // l = sum_c exp2(m_c - m) l_c
  for (int g0 = 0; g0 < G; g0 += NT / 32) {
    const int g = g0 + tid / 32, l32 = tid & 31;
    if (g < G) {
      float m = -INFINITY;
      for (int c = l32; c < NC; c += 32) m = fmaxf(m, wch[g * NCM + c]);
#pragma unroll
      for (int o = 16; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 32));
      float l = 0.f;
      for (int c = l32; c < NC; c += 32) {
        const float wc = exp2f(wch[g * NCM + c] - m);
        wch[g * NCM + c] = wc;
        l += wc * lch[g * NCM + c];
      }
#pragma unroll
      for (int o = 16; o > 0; o >>= 1) l += __shfl_xor(l, o, 32);
      if (l32 == 0) {
        lsum[g] = l;
        gate[g] = 1.f / (1.f + expf(-a.beta[hq0 + g]));
      }
    }
  }
  __syncthreads();

  T* out = static_cast<T*>(a.out) + ((int64_t)b * a.Hq + hq0) * DV;
  for (int x = tid; x < G * 32; x += NT) {
    const int g = x / 32, cs = x % 32, col = 32 * slab + cs;
    float o = 0.f;
    if (staged)
      for (int c = 0; c < NC; ++c) o += wch[g * NCM + c] * os[(c * G + g) * 32 + cs];
    else
      for (int c = 0; c < NC; ++c) o += wch[g * NCM + c] * part[(c * G + g) * (DV + 2) + 2 + col];
    const float r = a.retr[((int64_t)unit * G + g) * DV + col];
    const float den = a.rden[unit * G + g];
    out[g * DV + col] = from_f32<T>(gate[g] * (r / den) + (1.f - gate[g]) * (o / lsum[g]));
  }
}

template <typename T, int DK, int DV>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
  const unsigned units = (unsigned)(a.B * a.Hkv);
  // groups of up to 4 query heads take the instantiation with LDS for 4,
  // so more workgroups share a CU
  const unsigned grid = units * (unsigned)a.n_chunks + units * (unsigned)(DV / 32);
  if (a.G <= 4)
    hipLaunchKernelGGL((decode_partial_kernel<T, DK, DV, 4>), dim3(grid), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_partial_kernel<T, DK, DV, kDecodeMaxGroup>), dim3(grid),
                       dim3(256), 0, stream, a);
  hipLaunchKernelGGL((decode_combine_kernel<T, DK, DV>), dim3(units * (unsigned)(DV / 32)),
                     dim3(kDecodeNT), 0, stream, a);
  return hipGetLastError();
}

template <typename T, int DK>
hipError_t launch_decode_v(int dv, const DecodeArgs& a, hipStream_t stream) {
  switch (dv) {
    case 32: return launch_decode_t<T, DK, 32>(a, stream);
    case 64: return launch_decode_t<T, DK, 64>(a, stream);
    case 128: return launch_decode_t<T, DK, 128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
hipError_t launch_decode_kv(int dk, int dv, const DecodeArgs& a, hipStream_t stream) {
  switch (dk) {
    case 32: return launch_decode_v<T, 32>(dv, a, stream);
    case 64: return launch_decode_v<T, 64>(dv, a, stream);
    case 128: return launch_decode_v<T, 128>(dv, a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode(int dtype, int d, const DecodeArgs& a, hipStream_t stream) {
  return launch_decode_kv(dtype, d, d, a, stream);
}

hipError_t launch_decode_kv(int dtype, int dk, int dv, const DecodeArgs& a, hipStream_t stream) {
  return dtype == kBF16 ? launch_decode_kv<bf16>(dk, dv, a, stream)
                        : launch_decode_kv<float>(dk, dv, a, stream);
}

}  // namespace infini

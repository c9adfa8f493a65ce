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
//   partial: per (batch, KV head, chunk of 256 cache rows), the grouped query
//            heads' scores, chunk maximum, exp2 weights, their sum and the
//            weighted value sum (split over key groups, then reduced in LDS);
//            the workgroup whose chunk holds row pos also appends the token's
//            key and value to the cache (no workgroup reads that row from the
//            cache in this step: it takes the new key/value directly);
//   combine: per (batch, KV head), the chunks merged by their maxima, the
//            retrieval from the float state, the gate, the output row.
// The fold of a full segment into (M, z) reuses the recurrence kernels
// (api.hip).
#include "common.hpp"
#include "kernels.hpp"

namespace infini {

namespace {

constexpr int kDecodeKC = 256;  // cache rows per partial workgroup
constexpr int kDecodeNT = 256;  // threads per workgroup

template <typename T, int D>
__global__ __launch_bounds__(kDecodeNT) void decode_partial_kernel(DecodeArgs a) {
  constexpr int KC = kDecodeKC, NT = kDecodeNT, GM = kDecodeMaxGroup, C8 = D / 8;
  __shared__ float qs[GM * D];  // the group's queries, scaled by log2(e) / sqrt(d)
  __shared__ float ps[GM * KC]; // scores, then exp2 weights
  __shared__ float ov[NT * 8];  // per key-group partial value sums
  __shared__ float hm[GM], hl[GM];

  const int tid = threadIdx.x;
  const int G = a.G;
  const int unit = blockIdx.x / a.n_chunks, ch = blockIdx.x % a.n_chunks;
  const int b = unit / a.Hkv, j = unit % a.Hkv;
  const int t0 = ch * KC;
  const int n = min(KC, a.pos + 1 - t0);  // rows of this chunk, >= 1
  const T* q = static_cast<const T*>(a.q) + ((int64_t)b * a.Hq + (int64_t)j * G) * D;
  const T* knew = static_cast<const T*>(a.k) + (int64_t)unit * D;
  const T* vnew = static_cast<const T*>(a.v) + (int64_t)unit * D;
  const T* kc = static_cast<const T*>(a.k_cache) + (int64_t)unit * a.seg_len * D;
  const T* vc = static_cast<const T*>(a.v_cache) + (int64_t)unit * a.seg_len * D;

  for (int x = tid; x < G * D; x += NT) qs[x] = to_f32<T>(q[x]) * a.scale_log2;
  __syncthreads();

  // scores: one cache row per thread
  {
    float s[GM];
#pragma unroll
    for (int g = 0; g < GM; ++g) s[g] = 0.f;
    if (tid < n) {
      const int t = t0 + tid;
      const T* row = t == a.pos ? knew : kc + (int64_t)t * D;
#pragma unroll
      for (int c = 0; c < C8; ++c) {
        const frag_t<T> kv = load8<T>(row + 8 * c);
#pragma unroll
        for (int g = 0; g < GM; ++g)
          if (g < G) {
#pragma unroll
            for (int e = 0; e < 8; ++e) s[g] += to_f32<T>(kv[e]) * qs[g * D + 8 * c + e];
          }
      }
    }
#pragma unroll
    for (int g = 0; g < GM; ++g)
      if (g < G) ps[g * KC + tid] = tid < n ? s[g] : -INFINITY;
  }
  __syncthreads();

  // per head: chunk maximum, then exp2 weights and their sum (32 threads a head)
  for (int g0 = 0; g0 < G; g0 += NT / 32) {
    const int g = g0 + tid / 32, l32 = tid & 31;
    if (g < G) {
      float m = -INFINITY;
#pragma unroll
      for (int i = 0; i < KC / 32; ++i) m = fmaxf(m, ps[g * KC + l32 * (KC / 32) + i]);
#pragma unroll
      for (int o = 16; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 32));
      float l = 0.f;
#pragma unroll
      for (int i = 0; i < KC / 32; ++i) {
        const int x = g * KC + l32 * (KC / 32) + i;
        const float p = exp2f(ps[x] - m);  // -inf rows give 0
        ps[x] = p;
        l += p;
      }
#pragma unroll
      for (int o = 16; o > 0; o >>= 1) l += __shfl_xor(l, o, 32);
      if (l32 == 0) {
        hm[g] = m;
        hl[g] = l;
      }
    }
  }
  __syncthreads();

  // weighted value sums: (head, 8-column group) pairs, split over key groups
  const int npairs = G * C8;
  const int ks = max(1, NT / npairs);
  for (int p = tid; p < npairs * ks; p += NT) {
    const int pair = p % npairs, kg = p / npairs;
    const int g = pair / C8, c = pair % C8;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    for (int tt = kg; tt < n; tt += ks) {
      const int t = t0 + tt;
      const T* row = t == a.pos ? vnew : vc + (int64_t)t * D;
      const frag_t<T> vv = load8<T>(row + 8 * c);
      const float w = ps[g * KC + tt];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += w * to_f32<T>(vv[e]);
    }
    if (p < NT) {  // one slot per thread: npairs * ks <= NT when npairs <= NT
#pragma unroll
      for (int e = 0; e < 8; ++e) ov[p * 8 + e] = acc[e];
    }
  }
  __syncthreads();

  float* part = a.part + ((int64_t)unit * a.n_chunks + ch) * G * (D + 2);
  for (int x = tid; x < G * D; x += NT) {
    const int g = x / D, col = x % D, c = col / 8, e = col % 8;
    float o = 0.f;
    for (int kg = 0; kg < ks; ++kg) o += ov[(kg * npairs + g * C8 + c) * 8 + e];
    part[g * (D + 2) + 2 + col] = o;
  }
  if (tid < G) {
    part[tid * (D + 2)] = hm[tid];
    part[tid * (D + 2) + 1] = hl[tid];
  }

  // append the token to the cache
  if (t0 <= a.pos && a.pos < t0 + KC) {
    T* kw = static_cast<T*>(a.k_cache) + ((int64_t)unit * a.seg_len + a.pos) * D;
    T* vw = static_cast<T*>(a.v_cache) + ((int64_t)unit * a.seg_len + a.pos) * D;
    for (int x = tid; x < D; x += NT) {
      kw[x] = knew[x];
      vw[x] = vnew[x];
    }
  }
}

template <typename T, int D>
__global__ __launch_bounds__(kDecodeNT) void decode_combine_kernel(DecodeArgs a) {
  constexpr int NT = kDecodeNT, GM = kDecodeMaxGroup, NCM = kDecodeMaxChunks;
  __shared__ float sq[GM * D];    // sigma(q)
  __shared__ float wch[GM * NCM]; // chunk weights exp2(m_c - m) / l
  __shared__ float den[GM], gate[GM];

  const int tid = threadIdx.x;
  const int G = a.G, NC = a.n_chunks;
  const int unit = blockIdx.x;
  const int b = unit / a.Hkv, j = unit % a.Hkv;
  const int hq0 = j * G;
  const T* q = static_cast<const T*>(a.q) + ((int64_t)b * a.Hq + hq0) * D;
  const float* M = a.M + (int64_t)unit * D * D;
  const float* z = a.z + (int64_t)unit * D;
  const float* part = a.part + (int64_t)unit * NC * G * (D + 2);

  for (int x = tid; x < G * D; x += NT) sq[x] = feature_map(to_f32<T>(q[x]));
  __syncthreads();
  if (tid < G) {
    const int g = tid;
    float dp = 0.f;
    for (int k = 0; k < D; ++k) dp += sq[g * D + k] * z[k];
    den[g] = dp;
    gate[g] = 1.f / (1.f + expf(-a.beta[hq0 + g]));
    float m = -INFINITY;
    for (int c = 0; c < NC; ++c) m = fmaxf(m, part[(c * G + g) * (D + 2)]);
    float l = 0.f;
    for (int c = 0; c < NC; ++c) {
      const float w = exp2f(part[(c * G + g) * (D + 2)] - m);
      wch[g * NCM + c] = w;
      l += w * part[(c * G + g) * (D + 2) + 1];
    }
    for (int c = 0; c < NC; ++c) wch[g * NCM + c] /= l;
  }
  __syncthreads();

  T* out = static_cast<T*>(a.out) + ((int64_t)b * a.Hq + hq0) * D;
  for (int x = tid; x < G * D; x += NT) {
    const int g = x / D, col = x % D;
    float o = 0.f;
    for (int c = 0; c < NC; ++c) o += wch[g * NCM + c] * part[(c * G + g) * (D + 2) + 2 + col];
    float r = 0.f;
    for (int k = 0; k < D; ++k) r += sq[g * D + k] * M[(int64_t)k * D + col];
    out[x] = from_f32<T>(gate[g] * (r / den[g]) + (1.f - gate[g]) * o);
  }
}

template <typename T, int D>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
  const unsigned units = (unsigned)(a.B * a.Hkv);
  hipLaunchKernelGGL((decode_partial_kernel<T, D>), dim3(units * (unsigned)a.n_chunks),
                     dim3(kDecodeNT), 0, stream, a);
  hipLaunchKernelGGL((decode_combine_kernel<T, D>), dim3(units), dim3(kDecodeNT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(int dtype, int d, const DecodeArgs& a, hipStream_t stream) {
  if (dtype == kBF16) {
    switch (d) {
      case 32: return launch_decode_t<bf16, 32>(a, stream);
      case 64: return launch_decode_t<bf16, 64>(a, stream);
      case 128: return launch_decode_t<bf16, 128>(a, stream);
    }
  } else {
    switch (d) {
      case 32: return launch_decode_t<float, 32>(a, stream);
      case 64: return launch_decode_t<float, 64>(a, stream);
      case 128: return launch_decode_t<float, 128>(a, stream);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace infini

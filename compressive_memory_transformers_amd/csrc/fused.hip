// The whole forward in one pass for short segments: one workgroup per
// (batch, head) walks the segments in order and keeps the memory resident.
//
// "Infini-Attention" (AI Wiki), "What happens inside the Infini-attention
// block?" and "How does the compressive memory work?"; "Hugging Face
// Infini-Attention Reproduction Analysis", "Infini-Attention Mechanism",
// steps 1-6. For each segment s, with (M, z) the state left by segment s-1:
//   out  = g sigma(Q)M / (sigma(Q)z) + (1 - g) causal softmax(Q K^T / sqrt(d)) V
//   delta:  M += sigma(K)^T V - sigma(K)^T (sigma(K) M / (sigma(K) z))
//   linear: M += sigma(K)^T V
//   z += sum_t sigma(K_t)
//
// With segments no longer than d the split plan (a scan that writes the state
// before every segment, then a parallel attention that reads it back) moves
// the d x d state through memory once per segment, more than the segment's
// own Q, K and V. Here the state never leaves the chip: M lives in float
// registers, split into 32-column slabs, one per "update" wave; its bf16
// transpose sits in LDS for the matrix operands; z lives in LDS. The other
// half of the waves run the local attention, retrieval and gate of one
// 32-row query block each. Per segment:
//   1. the update waves store the segment's K and V (loaded into registers
//      during the previous segment) into LDS; the attention waves take their
//      Q rows; one barrier;
//   2. attention waves: S^T = K Q^T over the causal key blocks (online
//      softmax), O^T = V^T P^T, R^T = M^T sigma(Q)^T, and the rows
//      (1 - g)/l O + g/den R written out. Beside them the update waves stage
//      sigma(K) into LDS from the K rows still in their registers, with
//      den_t = sigma(K_t) . z and the column sums of sigma(K), wait for one
//      another on an LDS counter (the attention waves read none of it and do
//      not wait), then, per 32-token block: P = sigma(K) M for their slab
//      (delta), M += sigma(K)^T V + sigma(K)^T (-P / den), with -P/den taken
//      from the accumulator straight into the second product's operand
//      (never through LDS, never V - P/den rounded as one value);
//   3. after a second barrier the update waves write their slab's new M^T to
//      LDS and z += column sums.
// All products run on bf16 MFMA with float accumulation; the state stays
// float. The arithmetic is the split plan's, operand for operand.
#include "common.hpp"
#include "kernels.hpp"
#include "lds_tile.hpp"

namespace infini {

namespace {

template <int D, int RULE>
__global__ __launch_bounds__(D / 32 * 128) void fused_kernel(FusedArgs a) {
  constexpr int NB = D / 32;        // 32-wide blocks of d (and of the segment)
  constexpr int NT = NB * 128;      // threads: NB attention + NB update waves
  constexpr int NC = D / 16;        // 16-wide k chunks of d
  constexpr int CPR = D / 8;        // 16-byte chunks of a row
  constexpr int MTS = D + 8;        // row stride of M^T in LDS
  constexpr int PF = 2 * NB;        // 16-byte K and V chunks per update-wave thread
  constexpr bool DELTA = RULE == kRuleDelta;
  // Who stages sigma(K): with two waves per SIMD (d = 128) every wave stages
  // a share from LDS, so the VALU work spreads over all eight; with one wave
  // per SIMD (d = 64) the update waves stage alone from the K rows in their
  // registers while the attention waves run.
  constexpr bool ALL_STAGE = D == 128;
  constexpr int RED_ROWS = ALL_STAGE ? 32 : NB;  // column-sum partial rows
  static_assert(NT / CPR == 32, "32 rows per staging pass");
  static_assert((NB * 64) % (16 * CPR) == 0, "prefetch rows keep their swizzle");

  __shared__ __align__(1024) bf16 Ks[D * D];  // K of the segment, K layout
  __shared__ __align__(1024) bf16 Vs[D * D];  // V, V layout
  __shared__ __align__(1024) bf16 Ph[D * D];  // sigma(K), K layout
  __shared__ __align__(16) bf16 Mt[D * MTS];  // M^T (bf16), [value][key]
  __shared__ __align__(16) float red[RED_ROWS * D];  // column-sum partials
  __shared__ uint32_t staged;                 // update waves done staging, over all segments
  __shared__ float rden_s[D];                 // 1 / (sigma(K_t) . z) per token, 0 past the end
  __shared__ float zs[D];                     // z

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i = lane & 31, h = lane >> 5;
  const int unit = blockIdx.x;  // b * H + head
  const bool attn_wave = w < NB;
  const int head = unit % a.H;
  const int64_t L = a.L;
  const int N = a.seg_len;
  const int S = (int)((L + N - 1) / N);
  const bf16* Q = static_cast<const bf16*>(a.q) + (int64_t)unit * L * D;
  const bf16* K = static_cast<const bf16*>(a.k) + (int64_t)unit * L * D;
  const bf16* V = static_cast<const bf16*>(a.v) + (int64_t)unit * L * D;
  bf16* O = static_cast<bf16*>(a.out) + (int64_t)unit * L * D;
  const float c = a.scale_log2;
  const float g = 1.f / (1.f + __expf(-a.beta[head]));

  const uint32_t ko = 2 * (i * D + 8 * (h ^ swz_k<D>(i)));  // row reads of a K-layout tile
  if (tid < D) zs[tid] = a.z_in[(int64_t)unit * D + tid];  // attention-wave threads
  if (tid == 0) staged = 0u;

  // M in float goes through LDS on its way in and out (rows 0 .. d/2 - 1 in
  // the K buffer, the rest in the V buffer, both free then), so every global
  // access is a whole 16-byte piece of a row
  auto mstage = [&](int row) -> float* {
    return reinterpret_cast<float*>(row < D / 2 ? Ks : Vs) + (row % (D / 2)) * D;
  };
  {
    const float* Mi = a.M_in + (int64_t)unit * D * D;
#pragma unroll
    for (int k = 0; k < D * D / 4 / NT; ++k) {
      const int ch = tid + NT * k, row = ch / (D / 4), c4 = ch % (D / 4);
      *reinterpret_cast<f32x4*>(mstage(row) + 4 * c4) =
          *reinterpret_cast<const f32x4*>(Mi + row * D + 4 * c4);
    }
  }
  __syncthreads();

  // sigma(K) of the segment into Ph, 1 / den_t into rden_s, column-sum
  // partials into red, by every thread from the K tile in LDS (32 rows per
  // pass): the ALL_STAGE staging
  auto stage_all = [&](int n) {
    const int tr = tid / CPR, cc = tid % CPR;
    float zc[8], cs[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      zc[e] = zs[8 * cc + e];
      cs[e] = 0.f;
    }
#pragma unroll
    for (int p = 0; p < NB; ++p) {
      const int t = tr + 32 * p;
      const bf16x8 kv = load8<bf16>(Ks + t * D + 8 * (cc ^ swz_k<D>(t)));
      bf16x8 y;
      float dp = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float f = t < n ? feature_map((float)kv[e]) : 0.f;
        y[e] = (bf16)f;
        dp += f * zc[e];
        cs[e] += f;
      }
      store8<bf16>(Ph + t * D + 8 * (cc ^ swz_k<D>(t)), y);
      const float den = row_sum<CPR>(dp);
      if (cc == 0) rden_s[t] = t < n ? 1.f / den : 0.f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) red[tr * D + 8 * cc + e] = cs[e];
  };
  // every staging wave counts itself in on `staged` once its LDS stores are
  // done (release); the update waves then read the count (acquire) until all
  // staging waves of the segment are in. The wait is bounded: no staging wave
  // waits on anything before it counts itself in.
  auto count_in = [&]() {
    if (lane == 0)
      __hip_atomic_fetch_add(&staged, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
  };

  // The two roles run separate loops (so neither holds the other's
  // registers), with the same two barriers per segment:
  //   B1 the segment's K, V in LDS, and M^T and z of the state before it;
  //   B3 the segment's reads of Ks, Vs, Ph, Mt, red done.
  // Between them the update waves alone also wait for sigma(K) to be staged
  // (the LDS counter `staged`); the attention waves, which read none of it,
  // run on.
  if (attn_wave) {
    // ---- attention, retrieval and gate for query block w ----
    bf16x8 qf[NC], qn[NC];
    // row 32 w + i, 16-byte chunks 2 cc + h, by buffer loads over the
    // segment's valid rows (rows past its end read 0)
    const uint32_t qoff = (uint32_t)((32 * w + i) * D + 8 * h) * 2;
    auto load_q = [&](int s, bf16x8* dst) {
      const int64_t t0 = (int64_t)s * N;
      const uint32_t bytes = (uint32_t)min<int64_t>(N, L - t0) * D * 2;
      const __amdgpu_buffer_rsrc_t rq = raw_rsrc(Q + t0 * D, bytes);
#pragma unroll
      for (int cc = 0; cc < NC; ++cc)
        dst[cc] = __builtin_bit_cast(bf16x8,
                                     __builtin_amdgcn_raw_buffer_load_b128(rq, qoff, 32 * cc, 0));
    };
    uint32_t vo[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) vo[b] = tr_offset<D>(lane, b);
    load_q(0, qn);
    __syncthreads();  // the update waves' slabs are read
    for (int s = 0; s < S; ++s) {
      const int64_t t0 = (int64_t)s * N;
      const int n = (int)min<int64_t>(N, L - t0);
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) qf[cc] = qn[cc];
      __syncthreads();  // B1
      if (s + 1 < S) load_q(s + 1, qn);
      if constexpr (ALL_STAGE) {
        stage_all(n);
        count_in();
      }
      const int row = 32 * w + i;
      if (32 * w < n) {
        f32x16 oacc[NB];
#pragma unroll
        for (int db = 0; db < NB; ++db) oacc[db] = zero16();
        float m_run = -INFINITY, l_run = 0.f;
        for (int kb = 0; kb <= w; ++kb) {
          f32x16 sa = zero16();
#pragma unroll
          for (int cc = 0; cc < NC; ++cc)
            mma32(sa, load8<bf16>(lds_at(Ks, (ko ^ (32u * cc)) + 2 * 32 * kb * D)), qf[cc]);
          if (kb == w) {
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (32 * kb + acc_row(r, h) > row) sa[r] = -INFINITY;
          }
          float mx = -INFINITY;
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sa[r]);
          mx = xhalf_max(mx);  // key 32 kb is visible to every row: finite
          // lazy rescale: the reference only moves when a score exceeds it by
          // more than 2^8 (so exp2 arguments stay <= 8); numerator and
          // denominator share the reference either way
          if (__any((mx - m_run) * c > 8.f)) {
            const float m_new = fmaxf(m_run, mx);
            const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c);
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < NB; ++db)
#pragma unroll
              for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
            m_run = m_new;
          }
          const float mc = m_run * c;
          bf16x8 pf[2];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[r], c, -mc));
            pf[r >> 3][r & 7] = (bf16)p;
            l_run += (float)pf[r >> 3][r & 7];
          }
#pragma unroll
          for (int db = 0; db < NB; ++db)
#pragma unroll
            for (int pc = 0; pc < 2; ++pc)
              mma32(oacc[db], tr_frag<D>(Vs, vo[db], 2 * kb + pc), pf[pc]);
        }
        const float l = xhalf_sum(l_run);
        if (a.lse != nullptr && h == 0 && row < n)
          a.lse[(int64_t)unit * L + t0 + row] = m_run * c + __log2f(l);
        // retrieval from the unscaled sigma(Q) into its own accumulator;
        // g / den applies in float at the end
        bf16x8 sf[NC];
        float dpv[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int cc = 0; cc < NC; ++cc)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float sg = feature_map((float)qf[cc][e]);
            sf[cc][e] = (bf16)sg;
            dpv[e & 3] += sg * zs[16 * cc + 8 * h + e];
          }
        f32x16 racc[NB];
#pragma unroll
        for (int db = 0; db < NB; ++db) {
          racc[db] = zero16();
#pragma unroll
          for (int cc = 0; cc < NC; ++cc)
            mma32(racc[db], load8<bf16>(Mt + (32 * db + i) * MTS + 16 * cc + 8 * h), sf[cc]);
        }
        const float den = xhalf_sum((dpv[0] + dpv[1]) + (dpv[2] + dpv[3]));
        const float ca = (1.f - g) / l, cm = g / den;
        if (row < n) {
          bf16* orow = O + (t0 + row) * D;
#pragma unroll
          for (int db = 0; db < NB; ++db)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
              bf16x4 y;
#pragma unroll
              for (int j = 0; j < 4; ++j)
                y[j] = (bf16)__builtin_fmaf(oacc[db][4 * rq + j], ca, racc[db][4 * rq + j] * cm);
              store4<bf16>(orow + 32 * db + 8 * rq + 4 * h, y);
            }
        }
      }
      __syncthreads();  // B3
      if (tid < D) {    // z of the next state
        float cs = 0.f;
#pragma unroll
        for (int u = 0; u < RED_ROWS; ++u) cs += red[u * D + tid];
        zs[tid] += cs;
      }
    }
    if (tid < D) a.z_out[(int64_t)unit * D + tid] = zs[tid];
  } else {
    // ---- the memory update of value columns 32 vb .. + 31 ----
    const int vb = w - NB;
    const int ut = tid - NB * 64;
    f32x16 macc[NB];  // M rows 32 ib + acc_row(r, h), column 32 vb + i
#pragma unroll
    for (int ib = 0; ib < NB; ++ib)
#pragma unroll
      for (int r = 0; r < 16; ++r) macc[ib][r] = mstage(32 * ib + acc_row(r, h))[32 * vb + i];
    auto write_mt = [&]() {
#pragma unroll
      for (int ib = 0; ib < NB; ++ib)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          bf16x4 y;
#pragma unroll
          for (int j = 0; j < 4; ++j) y[j] = (bf16)macc[ib][4 * rq + j];
          store4<bf16>(Mt + (32 * vb + i) * MTS + 32 * ib + 8 * rq + 4 * h, y);
        }
    };
    write_mt();
    __syncthreads();  // every slab read before the first K and V overwrite the staging
    const uint32_t vo = tr_offset<D>(lane, vb);
    uint32_t po0[NB], po1[NB];  // transposed reads of sigma(K): key dims of block ib
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      po0[b] = tr_offset_k<D>(lane, b, 0);
      po1[b] = tr_offset_k<D>(lane, b, 1);
    }
    // chunk k of this thread: row ut / CPR + RSTEP k, 16-byte chunk ut % CPR;
    // buffer loads over the segment's valid rows (rows past its end read 0)
    constexpr int RSTEP = NB * 64 / CPR;
    const uint32_t kvoff = (uint32_t)((ut / CPR) * D + 8 * (ut % CPR)) * 2;
    frag_t<bf16> kpre[PF], vpre[PF];
    auto load_kv = [&](int s) {
      const int64_t t0 = (int64_t)s * N;
      const uint32_t bytes = (uint32_t)min<int64_t>(N, L - t0) * D * 2;
      const __amdgpu_buffer_rsrc_t rk = raw_rsrc(K + t0 * D, bytes);
      const __amdgpu_buffer_rsrc_t rv = raw_rsrc(V + t0 * D, bytes);
#pragma unroll
      for (int k = 0; k < PF; ++k) {
        kpre[k] = __builtin_bit_cast(
            bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rk, kvoff, k * RSTEP * D * 2, 0));
        vpre[k] = __builtin_bit_cast(
            bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rv, kvoff, k * RSTEP * D * 2, 0));
      }
    };
    load_kv(0);
    for (int s = 0; s < S; ++s) {
      const int64_t t0 = (int64_t)s * N;
      const int n = (int)min<int64_t>(N, L - t0);
      {
        // the rows RSTEP apart share their swizzles (period 16 in the row)
        const int r = ut / CPR, cc = ut % CPR;
        bf16* kd = Ks + r * D + 8 * (cc ^ swz_k<D>(r));
        bf16* vd = Vs + r * D + 8 * (cc ^ swz_v<D>(r));
#pragma unroll
        for (int k = 0; k < PF; ++k) {
          store8<bf16>(kd + k * RSTEP * D, kpre[k]);
          store8<bf16>(vd + k * RSTEP * D, vpre[k]);
        }
      }
      __syncthreads();  // B1
      if constexpr (ALL_STAGE) {
        stage_all(n);
      } else {
        // sigma(K) into Ph from the K rows in registers (rows r + RSTEP k,
        // 16-byte chunk cc), 1 / den_t into rden_s (the 8-element partial dot
        // in order, then summed over the row's CPR lanes), and the column
        // sums: over this thread's rows, then over the lanes of its chunk,
        // one row of red per wave
        const int r = ut / CPR, cc = ut % CPR;
        float zc[8], cs[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          zc[e] = zs[8 * cc + e];
          cs[e] = 0.f;
        }
        bf16* pd = Ph + r * D + 8 * (cc ^ swz_k<D>(r));
#pragma unroll
        for (int k = 0; k < PF; ++k) {
          const int t = r + k * RSTEP;
          bf16x8 y;
          float dp = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float f = t < n ? feature_map((float)kpre[k][e]) : 0.f;
            y[e] = (bf16)f;
            dp += f * zc[e];
            cs[e] += f;
          }
          store8<bf16>(pd + k * RSTEP * D, y);
          const float den = row_sum<CPR>(dp);
          if (cc == 0) rden_s[t] = t < n ? 1.f / den : 0.f;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
#pragma unroll
          for (int off = CPR; off < 32; off *= 2) cs[e] += __shfl_xor(cs[e], off);
          cs[e] = xhalf_sum(cs[e]);
        }
        if (lane < CPR) {
#pragma unroll
          for (int e = 0; e < 8; ++e) red[vb * D + 8 * lane + e] = cs[e];
        }
      }
      if (s + 1 < S) load_kv(s + 1);  // the K rows in registers are consumed
      count_in();
      {
        const uint32_t target = (uint32_t)(ALL_STAGE ? 2 * NB : NB) * (uint32_t)(s + 1);
        for (int spin = 0; spin < (1 << 22); ++spin) {
          const uint32_t v =
              __hip_atomic_load(&staged, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP);
          if ((int32_t)(v - target) >= 0) break;
          __builtin_amdgcn_s_sleep(1);
        }
      }
      // M += sigma(K)^T V (+ sigma(K)^T (-P / den), delta), one 32-token block
      // at a time. -P / den enters as the B operand straight from P's
      // accumulator: chunk p of 16 tokens, element e = token 16 p +
      // 8 (e / 4) + 4 h + e % 4, the accumulator's row order, which the
      // transposed reads of sigma(K) and V follow too.
#pragma unroll
      for (int tb = 0; tb < NB; ++tb) {
        f32x16 pacc;
        if constexpr (DELTA) {
          pacc = zero16();
#pragma unroll
          for (int cc = 0; cc < NC; ++cc)
            mma32(pacc, load8<bf16>(lds_at(Ph, (ko ^ (32u * cc)) + 2 * 32 * tb * D)),
                  load8<bf16>(Mt + (32 * vb + i) * MTS + 16 * cc + 8 * h));
        }
#pragma unroll
        for (int pc = 0; pc < 2; ++pc) {
          const int p = 2 * tb + pc;
          bf16x8 df;
          if constexpr (DELTA) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              df[e] = (bf16)(-pacc[8 * pc + e] * rden_s[32 * tb + acc_row(8 * pc + e, h)]);
          }
          const bf16x8 vf = tr_frag<D>(Vs, vo, p);
#pragma unroll
          for (int ib = 0; ib < NB; ++ib) {
            const bf16x8 af = tr_frag_k<D>(Ph, po0[ib], po1[ib], p);
            mma32(macc[ib], af, vf);
            if constexpr (DELTA) mma32(macc[ib], af, df);
          }
        }
      }
      __syncthreads();  // B3
      write_mt();
    }
#pragma unroll
    for (int ib = 0; ib < NB; ++ib)
#pragma unroll
      for (int r = 0; r < 16; ++r) mstage(32 * ib + acc_row(r, h))[32 * vb + i] = macc[ib][r];
  }
  __syncthreads();  // the final M is staged (the last segment's reads ended at B3)
  {
    float* Mo = a.M_out + (int64_t)unit * D * D;
#pragma unroll
    for (int k = 0; k < D * D / 4 / NT; ++k) {
      const int ch = tid + NT * k, row = ch / (D / 4), c4 = ch % (D / 4);
      *reinterpret_cast<f32x4*>(Mo + row * D + 4 * c4) =
          *reinterpret_cast<const f32x4*>(mstage(row) + 4 * c4);
    }
  }
}

template <int D>
hipError_t launch_fused_d(int rule, const FusedArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)a.units), block(D / 32 * 128);
  if (rule == kRuleDelta)
    hipLaunchKernelGGL((fused_kernel<D, kRuleDelta>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((fused_kernel<D, kRuleLinear>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace

bool fused_supported(int dtype, int d, int64_t seg_len, int64_t Hq, int64_t Hkv) {
  return dtype == kBF16 && (d == 64 || d == 128) && Hq == Hkv && seg_len <= d;
}

hipError_t launch_fused(int d, int rule, const FusedArgs& a, hipStream_t stream) {
  switch (d) {
    case 64: return launch_fused_d<64>(rule, a, stream);
    case 128: return launch_fused_d<128>(rule, a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace infini

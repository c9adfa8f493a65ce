// Backward pass of the Infini-attention block: gradients of out, M_final and
// z_final with respect to Q, K, V, beta, M0 and z0.
//
// "Infini-Attention" (AI Wiki), "How is an Infini-attention model trained?":
// gradients flow through the memory recurrence from segment to segment, as
// in truncated backpropagation through time; one call is the window. The
// derivation is the chain rule through each step of the forward ("What
// happens inside the Infini-attention block?", "How does the compressive
// memory work?"), in reverse order:
//
//   out = g A_mem + (1 - g) A_dot, g = sigmoid(beta_h):
//     dg = sum dout . (A_mem - A_dot) = sum dout . (A_mem - out) / (1 - g)
//   A_mem = X M / (X z), X = sigma(Q):
//     dn = g dout / den, dden = -g (dout . A_mem) / den,
//     dX = dn M^T + dden z^T, dM_{s-1} += X^T dn, dz_{s-1} += X^T dden
//   A_dot = softmax(Q K^T / sqrt(d)) V (causal): the usual softmax gradient
//     with delta_t = dA_dot,t . A_dot,t = dout_t . out_t - g dout_t . A_mem,t
//   update, Phi = sigma(K): z_s = z_{s-1} + sum Phi_t gives dPhi += dz_s;
//     linear M_s = M_{s-1} + Phi^T V: dV += Phi dM_s, dPhi += V dM_s^T;
//     delta  M_s = M_{s-1} + Phi^T U, U = V - P / c, P = Phi M_{s-1},
//     c = Phi z_{s-1}: dU = Phi dM_s, dV += dU, dP = -dU / c,
//     dc = (dU . P / c) / c, dPhi += U dM_s^T + dP M_{s-1}^T + dc z_{s-1}^T,
//     dM_{s-1} += Phi^T dP (= A_s dM_s), dz_{s-1} += Phi^T dc.
//
// The host plan (api.hip) strings these together with the batched matrix
// product below for every d x d product and the kernels here for the
// row-wise steps, the local attention, the dz recurrence and the outputs.
// The recurrence of dM runs in float whatever the element type: with a small
// z_{s-1} the delta rule's transition I + A_s has large entries, and bf16
// operands there would be amplified into the state gradients.
#include "common.hpp"
#include "kernels.hpp"
#include "lds_tile.hpp"

namespace infini {

namespace {

// sigma'(x): 1 above zero, e^x at or below (continuous at 0).
__device__ __forceinline__ float feature_map_grad(float x) {
  return x > 0.f ? 1.f : __builtin_amdgcn_exp2f(x * kLog2e);
}

__device__ __forceinline__ float gate_of(const float* beta, int h) {
  return 1.f / (1.f + __expf(-beta[h]));
}

// ---- batched matrix product ---------------------------------------------------
//
// 64 x 64 tile of C per workgroup (four waves of 32 x 32), K in steps of 32.
// op(A) is staged as [m][k], op(B) as [n][k], both with k contiguous, so that
// each MFMA operand is one 16-byte (bf16) or 32-byte (float) LDS read; a
// transposed operand is transposed while it is stored.
template <typename T>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs g) {
  constexpr int TM = 64, TN = 64, TK = 32, LS = TK + pad16<T>();
  __shared__ __align__(16) T As[TM * LS];
  __shared__ __align__(16) T Bs[TN * LS];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int i = lane & 31, h = lane >> 5;
  const int ntn = (g.N + TN - 1) / TN;
  const int64_t n_tiles_m = (g.M + TM - 1) / TM;
  const int64_t per_batch = n_tiles_m * ntn;
  const int64_t x = blockIdx.x;
  const int batch = (int)(x / per_batch);
  const int tile = (int)(x % per_batch);
  const int m0 = (tile / ntn) * TM, n0 = (tile % ntn) * TN;
  const int hi = batch / g.S, lo = batch % g.S;
  int Mv = g.M, Kv = g.K;
  if (g.clip != 0) {
    const int64_t rows = min<int64_t>(g.seg_len, g.L - (int64_t)lo * g.seg_len);
    if (g.clip == 1) Mv = (int)min<int64_t>(Mv, rows); else Kv = (int)min<int64_t>(Kv, rows);
  }
  if (m0 >= Mv) return;  // uniform
  const T* A = static_cast<const T*>(g.A) + (int64_t)(hi / g.a_div) * g.a_hi + (int64_t)lo * g.a_lo;
  const T* B = static_cast<const T*>(g.B) + (int64_t)(hi / g.b_div) * g.b_hi + (int64_t)lo * g.b_lo;
  float* C = g.C + (int64_t)(hi / g.c_div) * g.c_hi + (int64_t)lo * g.c_lo;

  const int wm = w >> 1, wn = w & 1;
  f32x16 acc = zero16();
  for (int k0 = 0; k0 < Kv; k0 += TK) {
    {  // A -> As[m][k]
      frag_t<T> val = zero_frag<T>();
      if (!g.ta) {
        const int r = tid >> 2, kc = (tid & 3) * 8;
        if (m0 + r < Mv && k0 + kc < Kv) val = load8<T>(A + (int64_t)(m0 + r) * g.lda + k0 + kc);
        if (g.a_sigma)
#pragma unroll
          for (int e = 0; e < 8; ++e) val[e] = from_f32<T>(feature_map(to_f32<T>(val[e])));
        store8<T>(As + r * LS + kc, val);
      } else {
        const int kr = tid >> 3, mc = (tid & 7) * 8;
        if (k0 + kr < Kv && m0 + mc < Mv) val = load8<T>(A + (int64_t)(k0 + kr) * g.lda + m0 + mc);
        if (g.a_sigma && k0 + kr < Kv)
#pragma unroll
          for (int e = 0; e < 8; ++e) val[e] = from_f32<T>(feature_map(to_f32<T>(val[e])));
#pragma unroll
        for (int e = 0; e < 8; ++e) As[(mc + e) * LS + kr] = val[e];
      }
    }
    {  // B -> Bs[n][k]
      frag_t<T> val = zero_frag<T>();
      if (g.tb) {
        const int r = tid >> 2, kc = (tid & 3) * 8;
        if (n0 + r < g.N && k0 + kc < Kv) val = load8<T>(B + (int64_t)(n0 + r) * g.ldb + k0 + kc);
        store8<T>(Bs + r * LS + kc, val);
      } else {
        const int kr = tid >> 3, nc = (tid & 7) * 8;
        if (k0 + kr < Kv && n0 + nc < g.N) val = load8<T>(B + (int64_t)(k0 + kr) * g.ldb + n0 + nc);
#pragma unroll
        for (int e = 0; e < 8; ++e) Bs[(nc + e) * LS + kr] = val[e];
      }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < TK; kk += 16)
      mma32(acc, load8<T>(As + (32 * wm + i) * LS + kk + 8 * h),
            load8<T>(Bs + (32 * wn + i) * LS + kk + 8 * h));
    __syncthreads();
  }
  const int n = n0 + 32 * wn + i;
  if (n >= g.N) return;
  if (g.epi == 1) {
    const float* wv = g.epi_w + (int64_t)(hi / g.c_div) * g.w_hi + (int64_t)lo * g.w_lo;
    const float zn = g.epi_z[(int64_t)(hi / g.z_div) * g.z_hi + (int64_t)lo * g.z_lo + n];
    const T* xv = static_cast<const T*>(g.epi_x) + (int64_t)(hi / g.c_div) * g.c_hi +
                  (int64_t)lo * g.c_lo;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + 32 * wm + acc_row(r, h);
      if (m < Mv)
        C[(int64_t)m * g.ldc + n] = (g.alpha * acc[r] + wv[m] * zn) *
                                    feature_map_grad(to_f32<T>(xv[(int64_t)m * g.ldc + n]));
    }
    return;
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int m = m0 + 32 * wm + acc_row(r, h);
    if (m < Mv) {
      float* c = C + (int64_t)m * g.ldc + n;
      *c = g.alpha * acc[r] + (g.accumulate ? *c : 0.f);
    }
  }
}

// ---- row steps (one wave per row, lane l holds elements l, l + 64) -----------

template <int D> struct RowLanes {
  static constexpr int E = (D + 63) / 64;
  __device__ static bool ok(int lane, int e) { return 64 * e + lane < D; }
};

// Retrieval backward, per query row: with nm = sigma(q) M_{s-1} (the
// numerator of A_mem), writes delta, dg, dden and dn (element type).
// DK: the key width (q, z); DV: the value width (out, dout, nm, dn).
template <typename T, int DK, int DV>
__global__ __launch_bounds__(256) void retrieval_rows_kernel(BwdArgs a) {
  using RK = RowLanes<DK>;
  using R = RowLanes<DV>;
  const int lane = threadIdx.x & 63;
  const int G = a.Hq / a.Hkv;
  const int64_t rows = (int64_t)a.B * a.Hq * a.L;
  for (int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); row < rows;
       row += (int64_t)gridDim.x * 4) {
    const int64_t bh = row / a.L, t = row % a.L;
    const int hq = (int)(bh % a.Hq), b = (int)(bh / a.Hq);
    const int s = (int)(t / a.seg_len);
    const int64_t unit = (int64_t)b * a.Hkv + hq / G;
    const float* z = a.snapZ + (unit * a.S + s) * DK;
    const T* q = static_cast<const T*>(a.q) + row * DK;
    // The segment's first row attends to its own key alone, so A_dot = v_t
    // and out = g A_mem + (1 - g) v_t: that row reads v_t in place of its
    // output row and forms delta = (1 - g) dout . v_t and d(gate) =
    // dout . A_mem - dout . v_t exactly. From the stored output, whose
    // rounding would not cancel against (1 - g) dout . v_t in dS (exactly
    // zero there), the rounding would land whole in that row's dQ.
    const bool first = t % a.seg_len == 0;  // wave-uniform
    const T* o = first ? static_cast<const T*>(a.v) + (unit * a.L + t) * DV
                       : static_cast<const T*>(a.out) + row * DV;
    const T* dO = static_cast<const T*>(a.dout) + row * DV;
    const float* nm = a.nm + row * DV;
    float den = 0.f;
#pragma unroll
    for (int e = 0; e < RK::E; ++e)
      if (RK::ok(lane, e)) den += feature_map(to_f32<T>(q[64 * e + lane])) * z[64 * e + lane];
    den = wave_sum(den);
    float am[R::E], dov[R::E];
    float dam = 0.f, doo = 0.f;
#pragma unroll
    for (int e = 0; e < R::E; ++e) {
      am[e] = dov[e] = 0.f;
      if (R::ok(lane, e)) {
        const int c = 64 * e + lane;
        am[e] = nm[c] / den;
        dov[e] = to_f32<T>(dO[c]);
        dam += dov[e] * am[e];
        doo += dov[e] * to_f32<T>(o[c]);
      }
    }
    dam = wave_sum(dam);
    doo = wave_sum(doo);
    const float g = gate_of(a.beta, hq);
    T* dn = static_cast<T*>(a.dn) + row * DV;
#pragma unroll
    for (int e = 0; e < R::E; ++e)
      if (R::ok(lane, e)) dn[64 * e + lane] = from_f32<T>(g * dov[e] / den);
    if (lane == 0) {
      // first row: doo = dout . v_t
      a.delta[row] = first ? (1.f - g) * doo : doo - g * dam;
      a.dg[row] = first ? dam - doo : (dam - doo) / (1.f - g);
      a.dden[row] = -g * dam / den;
    }
  }
}

// e[unit][s][c] = sum over the segment's rows t (and the group's query heads
// when of_q) of w_t sigma(x_t[c]): the retrieval (x = q, w = dden) or the
// delta rule's (x = k, w = dc) part of dL/dz_{s-1}. Two stages, in a fixed
// order (no atomics): workgroup ch of a (unit, segment) sums rows
// [ch R, (ch + 1) R) of the segment's G n or n rows into part, then
// wsum_final adds the chunks.
constexpr int kWsumRows = 512;

template <typename T, int D>
__global__ __launch_bounds__(256) void wsum_partial_kernel(BwdArgs a, int of_q, int n_chunks) {
  constexpr int CG = D / 8, RL = 256 / CG;
  __shared__ float red[RL * D];
  const int tid = threadIdx.x, cg = tid % CG, rl = tid / CG;
  const int ch = blockIdx.x % n_chunks;
  const int64_t us = blockIdx.x / n_chunks;  // unit * S + s
  const int64_t unit = us / a.S;
  const int s = (int)(us % a.S);
  const int G = a.Hq / a.Hkv;
  const int64_t t0 = (int64_t)s * a.seg_len;
  const int n = (int)min<int64_t>(a.seg_len, a.L - t0);
  const int R = of_q ? G * n : n;
  const int r1 = min(R, (ch + 1) * kWsumRows);
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  const int64_t b = unit / a.Hkv, j = unit % a.Hkv;
  for (int r = ch * kWsumRows + rl; r < r1; r += RL) {
    int64_t row;  // row of the [.][L] tensor
    if (of_q)
      row = (b * a.Hq + j * G + r / n) * a.L + t0 + r % n;
    else
      row = unit * a.L + t0 + r;
    const T* x = static_cast<const T*>(of_q ? a.q : a.k) + row * D + 8 * cg;
    const float wv = (of_q ? a.dden : a.dc)[row];
    const frag_t<T> xv = load8<T>(x);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += wv * feature_map(to_f32<T>(xv[e]));
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[rl * D + 8 * cg + e] = acc[e];
  __syncthreads();
  if (tid < D) {
    float t = 0.f;
    for (int k = 0; k < RL; ++k) t += red[k * D + tid];
    a.wsum_part[((int64_t)us * n_chunks + ch) * D + tid] = t;
  }
}

template <int D>
__global__ __launch_bounds__(D) void wsum_final_kernel(BwdArgs a, int of_q, int n_chunks) {
  const int64_t us = blockIdx.x;
  float t = 0.f;
  for (int ch = 0; ch < n_chunks; ++ch) t += a.wsum_part[((int64_t)us * n_chunks + ch) * D + threadIdx.x];
  (of_q ? a.e_ret : a.e_upd)[us * D + threadIdx.x] = t;
}

// ---- local attention, one wave per row (small shapes and float) -----------
//
// P_tu = exp2(c q_t . k_u - lse_t), c = log2(e) / sqrt(d); dA_dot = (1 - g)
// dout; dS_tu = P_tu ((1 - g) dout_t . v_u - delta_t);
// dQ_t = sum_u dS_tu k_u / sqrt(d), dK_u = sum_t dS_tu q_t / sqrt(d),
// dV_u = sum_t P_tu (1 - g) dout_t.

// DK: the key width (q, k, dq and its retrieval part in nm); DV: the value
// width (v, dout).
template <typename T, int DK, int DV>
__global__ __launch_bounds__(256) void attn_dq_rows_kernel(BwdArgs a) {
  using R = RowLanes<DK>;
  using RV = RowLanes<DV>;
  const int lane = threadIdx.x & 63;
  const int G = a.Hq / a.Hkv;
  const float c = a.scale_log2, inv_sqrt_d = a.scale_log2 / kLog2e;
  const int64_t rows = (int64_t)a.B * a.Hq * a.L;
  for (int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); row < rows;
       row += (int64_t)gridDim.x * 4) {
    const int64_t bh = row / a.L, t = row % a.L;
    const int hq = (int)(bh % a.Hq), b = (int)(bh / a.Hq);
    const int64_t unit = (int64_t)b * a.Hkv + hq / G;
    const int64_t t0 = t / a.seg_len * a.seg_len;
    const float om = 1.f - gate_of(a.beta, hq);
    const float lse = a.lse[row], dl = a.delta[row];
    float qv[R::E], dov[RV::E], acc[R::E];
#pragma unroll
    for (int e = 0; e < R::E; ++e) {
      const bool ok = R::ok(lane, e);
      qv[e] = ok ? to_f32<T>(static_cast<const T*>(a.q)[row * DK + 64 * e + lane]) : 0.f;
      acc[e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < RV::E; ++e)
      dov[e] = RV::ok(lane, e)
                   ? to_f32<T>(static_cast<const T*>(a.dout)[row * DV + 64 * e + lane])
                   : 0.f;
    const T* K = static_cast<const T*>(a.k) + unit * a.L * DK;
    const T* V = static_cast<const T*>(a.v) + unit * a.L * DV;
    for (int64_t u = t0; u <= t; ++u) {
      float kv[R::E], sd = 0.f, dp = 0.f;
#pragma unroll
      for (int e = 0; e < R::E; ++e) {
        const bool ok = R::ok(lane, e);
        kv[e] = ok ? to_f32<T>(K[u * DK + 64 * e + lane]) : 0.f;
        sd += qv[e] * kv[e];
      }
#pragma unroll
      for (int e = 0; e < RV::E; ++e)
        dp += dov[e] * (RV::ok(lane, e) ? to_f32<T>(V[u * DV + 64 * e + lane]) : 0.f);
      sd = wave_sum(sd);
      dp = wave_sum(dp);
      const float p = __builtin_amdgcn_exp2f(c * sd - lse);
      const float ds = p * (om * dp - dl);
#pragma unroll
      for (int e = 0; e < R::E; ++e) acc[e] += ds * kv[e];
    }
    T* dq = static_cast<T*>(a.dq) + row * DK;
#pragma unroll
    for (int e = 0; e < R::E; ++e)
      if (R::ok(lane, e))
        dq[64 * e + lane] = from_f32<T>(acc[e] * inv_sqrt_d + a.nm[row * DK + 64 * e + lane]);
  }
}

template <typename T, int DK, int DV>
__global__ __launch_bounds__(256) void attn_dkdv_rows_kernel(BwdArgs a) {
  using R = RowLanes<DK>;
  using RV = RowLanes<DV>;
  const int lane = threadIdx.x & 63;
  const int G = a.Hq / a.Hkv;
  const float c = a.scale_log2, inv_sqrt_d = a.scale_log2 / kLog2e;
  const int64_t rows = (int64_t)a.B * a.Hkv * a.L;
  for (int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); row < rows;
       row += (int64_t)gridDim.x * 4) {
    const int64_t unit = row / a.L, u = row % a.L;
    const int64_t b = unit / a.Hkv, j = unit % a.Hkv;
    const int64_t t1 = min<int64_t>((u / a.seg_len + 1) * a.seg_len, a.L);
    float kv[R::E], vv[RV::E], dk[R::E], dv[RV::E];
#pragma unroll
    for (int e = 0; e < R::E; ++e) {
      kv[e] = R::ok(lane, e) ? to_f32<T>(static_cast<const T*>(a.k)[row * DK + 64 * e + lane])
                             : 0.f;
      dk[e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < RV::E; ++e) {
      vv[e] = RV::ok(lane, e) ? to_f32<T>(static_cast<const T*>(a.v)[row * DV + 64 * e + lane])
                              : 0.f;
      dv[e] = 0.f;
    }
    for (int hg = 0; hg < G; ++hg) {
      const int hq = (int)(j * G + hg);
      const int64_t bh = b * a.Hq + hq;
      const float om = 1.f - gate_of(a.beta, hq);
      const T* Q = static_cast<const T*>(a.q) + bh * a.L * DK;
      const T* dO = static_cast<const T*>(a.dout) + bh * a.L * DV;
      for (int64_t t = u; t < t1; ++t) {
        float qv[R::E], dov[RV::E], sd = 0.f, dp = 0.f;
#pragma unroll
        for (int e = 0; e < R::E; ++e) {
          qv[e] = R::ok(lane, e) ? to_f32<T>(Q[t * DK + 64 * e + lane]) : 0.f;
          sd += qv[e] * kv[e];
        }
#pragma unroll
        for (int e = 0; e < RV::E; ++e) {
          dov[e] = RV::ok(lane, e) ? to_f32<T>(dO[t * DV + 64 * e + lane]) : 0.f;
          dp += dov[e] * vv[e];
        }
        sd = wave_sum(sd);
        dp = wave_sum(dp);
        const float p = __builtin_amdgcn_exp2f(c * sd - a.lse[bh * a.L + t]);
        const float ds = p * (om * dp - a.delta[bh * a.L + t]);
#pragma unroll
        for (int e = 0; e < R::E; ++e) dk[e] += ds * qv[e];
#pragma unroll
        for (int e = 0; e < RV::E; ++e) dv[e] += p * om * dov[e];
      }
    }
#pragma unroll
    for (int e = 0; e < R::E; ++e)
      if (R::ok(lane, e)) a.dk_acc[row * DK + 64 * e + lane] = dk[e] * inv_sqrt_d;
#pragma unroll
    for (int e = 0; e < RV::E; ++e)
      if (RV::ok(lane, e)) a.dv_acc[row * DV + 64 * e + lane] = dv[e];
  }
}

// ---- update backward, per key row ----------------------------------------------
//
// Linear: dv_acc += du_buf (= Phi dM_s). Delta, with p_buf = Phi M_{s-1}:
// c = Phi . z_{s-1}, pred = P / c, U = V - pred (u_el), dU = du_buf,
// dv_acc += dU, dP = -dU / c (dp_el), dc = (dU . pred) / c.
// DK: the key width (k, z); DV: the value width (v, p_buf, du_buf, u_el,
// dp_el, dv_acc).
template <typename T, int DK, int DV>
__global__ __launch_bounds__(256) void update_rows_kernel(BwdArgs a) {
  using RK = RowLanes<DK>;
  using R = RowLanes<DV>;
  const int lane = threadIdx.x & 63;
  const int64_t rows = (int64_t)a.B * a.Hkv * a.L;
  for (int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); row < rows;
       row += (int64_t)gridDim.x * 4) {
    if (a.rule == kRuleLinear) {
#pragma unroll
      for (int e = 0; e < R::E; ++e)
        if (R::ok(lane, e))
          a.dv_acc[row * DV + 64 * e + lane] += a.du_buf[row * DV + 64 * e + lane];
      continue;
    }
    const int64_t unit = row / a.L, t = row % a.L;
    const int s = (int)(t / a.seg_len);
    const float* z = a.snapZ + (unit * a.S + s) * DK;
    float cc = 0.f;
#pragma unroll
    for (int e = 0; e < RK::E; ++e)
      if (RK::ok(lane, e))
        cc += feature_map(to_f32<T>(static_cast<const T*>(a.k)[row * DK + 64 * e + lane])) *
              z[64 * e + lane];
    cc = wave_sum(cc);
    float dcs = 0.f;
#pragma unroll
    for (int e = 0; e < R::E; ++e)
      if (R::ok(lane, e)) {
        const int64_t x = row * DV + 64 * e + lane;
        const float pred = a.p_buf[x] / cc;
        const float du = a.du_buf[x];
        static_cast<T*>(a.u_el)[x] = from_f32<T>(to_f32<T>(static_cast<const T*>(a.v)[x]) - pred);
        static_cast<T*>(a.dp_el)[x] = from_f32<T>(-du / cc);
        a.dv_acc[x] += du;
        dcs += du * pred;
      }
    dcs = wave_sum(dcs);
    if (lane == 0) a.dc[row] = dcs / cc;
  }
}

// For A_s = -Phi^T diag(1/c) Phi in float (the state gradient's transition):
// phi_f = sigma(K) and phic_f = sigma(K) / c, c = sigma(k) . z_{s-1}.
template <typename T, int D>
__global__ __launch_bounds__(256) void phi_rows_kernel(BwdArgs a) {
  using R = RowLanes<D>;
  const int lane = threadIdx.x & 63;
  const int64_t rows = (int64_t)a.B * a.Hkv * a.L;
  for (int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); row < rows;
       row += (int64_t)gridDim.x * 4) {
    const int64_t unit = row / a.L, t = row % a.L;
    const float* z = a.snapZ + (unit * a.S + t / a.seg_len) * D;
    float ph[R::E], cc = 0.f;
#pragma unroll
    for (int e = 0; e < R::E; ++e) {
      ph[e] = R::ok(lane, e)
                  ? feature_map(to_f32<T>(static_cast<const T*>(a.k)[row * D + 64 * e + lane]))
                  : 0.f;
      if (R::ok(lane, e)) cc += ph[e] * z[64 * e + lane];
    }
    cc = wave_sum(cc);
#pragma unroll
    for (int e = 0; e < R::E; ++e)
      if (R::ok(lane, e)) {
        a.phi_f[row * D + 64 * e + lane] = ph[e];
        a.phic_f[row * D + 64 * e + lane] = ph[e] / cc;
      }
  }
}

template <typename T>
__global__ __launch_bounds__(256) void round_kernel(T* dst, const float* src, int64_t n) {
  for (int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x; x < n; x += (int64_t)gridDim.x * 256)
    dst[x] = from_f32<T>(src[x]);
}

// ---- dz recurrence and outputs ---------------------------------------------------

// dz_s for every segment, last to first: dz_{s-1} = dz_s + e_ret_s + e_upd_s.
template <int D>
__global__ __launch_bounds__(D) void dz_scan_kernel(BwdArgs a) {
  const int c = threadIdx.x;
  const int64_t unit = blockIdx.x;
  float dz = a.dz_final ? a.dz_final[unit * D + c] : 0.f;
  for (int s = a.S - 1; s >= 0; --s) {
    const int64_t x = (unit * a.S + s) * D + c;
    a.dzs[x] = dz;
    dz += a.e_ret[x];
    if (a.rule == kRuleDelta) dz += a.e_upd[x];
  }
  a.dz0[unit * D + c] = dz;
}

// dK = dk_acc + (dphi + dc z_{s-1} + dz_s) sigma'(k) (DK wide), dV = dv_acc
// (DV wide; unless the fused update kernel already wrote it). Each thread takes eight consecutive elements of a row (16-byte
// stores of the outputs; every pointer is 16-byte aligned and the widths are
// multiples of 8), so the row and segment are decoded once per eight.
template <typename T, int DK, int DV>
__global__ __launch_bounds__(256) void kv_out_kernel(BwdArgs a) {
  constexpr int CK = DK / 8, CV = DV / 8;
  const int64_t rows = (int64_t)a.B * a.Hkv * a.L;
  const int64_t stride = (int64_t)gridDim.x * 256;
  const int64_t nk = rows * CK;
  for (int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x; x < nk; x += stride) {
    const int64_t row = x / CK;
    const int c = (int)(x % CK) * 8;
    const int64_t unit = row / a.L, t = row - unit * a.L;
    const int s = (int)(t / a.seg_len);
    const int64_t e = row * DK + c;
    const int64_t sx = (unit * a.S + s) * DK + c;
    const frag_t<float> dphi = load8<float>(a.dphi + e);
    const frag_t<float> dz = load8<float>(a.dzs + sx);
    const frag_t<float> acc = load8<float>(a.dk_acc + e);
    const frag_t<T> kv = load8<T>(static_cast<const T*>(a.k) + e);
    frag_t<float> zc;
    float dcr = 0.f;
    if (a.rule == kRuleDelta) {
      zc = load8<float>(a.snapZ + sx);
      dcr = a.dc[row];
    }
    frag_t<T> y;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float g = dphi[j] + dz[j];
      if (a.rule == kRuleDelta) g += dcr * zc[j];
      y[j] = from_f32<T>(acc[j] + g * feature_map_grad(to_f32<T>(kv[j])));
    }
    store8<T>(static_cast<T*>(a.dk) + e, y);
  }
  if (a.dv_final) return;  // the fused update kernel wrote dv
  const int64_t nv = rows * CV;
  for (int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x; x < nv; x += stride) {
    const frag_t<float> acc = load8<float>(a.dv_acc + 8 * x);
    frag_t<T> y;
#pragma unroll
    for (int j = 0; j < 8; ++j) y[j] = from_f32<T>(acc[j]);
    store8<T>(static_cast<T*>(a.dv) + 8 * x, y);
  }
}

// dbeta_h = g (1 - g) sum over the batch and the stream of dg, in two
// passes with a fixed order (no atomics): workgroup (h, b, c) sums positions
// [c kDbetaChunk, (c + 1) kDbetaChunk) of row (b, h) into dbeta_part, then
// one thread per head adds that head's partials in (b, c) order.
__global__ __launch_bounds__(256) void dbeta_partial_kernel(BwdArgs a, int n_ch) {
  __shared__ float part[4];
  const int c = blockIdx.x % n_ch;
  const int64_t hb = blockIdx.x / n_ch;  // hq * B + b
  const int hq = (int)(hb / a.B), b = (int)(hb % a.B);
  const float* dg = a.dg + ((int64_t)b * a.Hq + hq) * a.L;
  const int64_t t1 = min<int64_t>(a.L, (int64_t)(c + 1) * kDbetaChunk);
  float acc = 0.f;
#pragma unroll 4
  for (int64_t t = (int64_t)c * kDbetaChunk + threadIdx.x; t < t1; t += 256) acc += dg[t];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) a.dbeta_part[blockIdx.x] = (part[0] + part[1]) + (part[2] + part[3]);
}

__global__ __launch_bounds__(256) void dbeta_final_kernel(BwdArgs a, int n_ch) {
  const int n = a.B * n_ch;
  for (int hq = threadIdx.x; hq < a.Hq; hq += 256) {
    const float* p = a.dbeta_part + (int64_t)hq * n;
    float t = 0.f;
    for (int i = 0; i < n; ++i) t += p[i];
    const float g = gate_of(a.beta, hq);
    a.dbeta[hq] = t * g * (1.f - g);
  }
}

__global__ __launch_bounds__(256) void fill_kernel(float* p, float v, int64_t n) {
  for (int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x; x < n; x += (int64_t)gridDim.x * 256)
    p[x] = v;
}

unsigned row_grid(int64_t rows) {  // 4 rows per workgroup, grid-stride beyond
  const int64_t n = (rows + 3) / 4;
  return (unsigned)(n < 65536 ? n : 65536);
}
unsigned elem_grid(int64_t n) {
  const int64_t g = (n + 255) / 256;
  return (unsigned)(g < 65536 ? g : 65536);
}

// D: the key width; DV: the value width.
template <typename T, int D, int DV>
hipError_t launch_d(int which, const BwdArgs& a, int arg, hipStream_t s) {
  const int64_t qrows = (int64_t)a.B * a.Hq * a.L, krows = (int64_t)a.B * a.Hkv * a.L;
  const int64_t units = (int64_t)a.B * a.Hkv;
  switch (which) {
    case 0:
      hipLaunchKernelGGL((retrieval_rows_kernel<T, D, DV>), dim3(row_grid(qrows)), dim3(256), 0, s,
                         a);
      break;
    case 2: {
      const int G = a.Hq / a.Hkv;
      const int64_t n = a.seg_len < a.L ? a.seg_len : a.L;
      const int n_chunks = (int)(((arg ? G : 1) * n + kWsumRows - 1) / kWsumRows);
      hipLaunchKernelGGL((wsum_partial_kernel<T, D>), dim3((unsigned)(units * a.S * n_chunks)),
                         dim3(256), 0, s, a, arg, n_chunks);
      hipLaunchKernelGGL((wsum_final_kernel<D>), dim3((unsigned)(units * a.S)), dim3(D), 0, s, a,
                         arg, n_chunks);
      break;
    }
    case 3:
      hipLaunchKernelGGL((attn_dkdv_rows_kernel<T, D, DV>), dim3(row_grid(krows)), dim3(256), 0, s,
                         a);
      hipLaunchKernelGGL((attn_dq_rows_kernel<T, D, DV>), dim3(row_grid(qrows)), dim3(256), 0, s,
                         a);
      break;
    case 4:
      hipLaunchKernelGGL((update_rows_kernel<T, D, DV>), dim3(row_grid(krows)), dim3(256), 0, s, a);
      break;
    case 6:
      hipLaunchKernelGGL((phi_rows_kernel<T, D>), dim3(row_grid(krows)), dim3(256), 0, s, a);
      break;
    case 5:
      hipLaunchKernelGGL((dz_scan_kernel<D>), dim3((unsigned)units), dim3(D), 0, s, a);
      hipLaunchKernelGGL((kv_out_kernel<T, D, DV>), dim3(elem_grid(krows * (D > DV ? D : DV) / 8)),
                         dim3(256), 0, s, a);
      {
        const int n_ch = (int)((a.L + kDbetaChunk - 1) / kDbetaChunk);
        hipLaunchKernelGGL((dbeta_partial_kernel), dim3((unsigned)((int64_t)a.Hq * a.B * n_ch)),
                           dim3(256), 0, s, a, n_ch);
        hipLaunchKernelGGL((dbeta_final_kernel), dim3(1), dim3(256), 0, s, a, n_ch);
      }
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_v(int dv, int which, const BwdArgs& a, int arg, hipStream_t s) {
  switch (dv) {
    case 32: return launch_d<T, D, 32>(which, a, arg, s);
    case 64: return launch_d<T, D, 64>(which, a, arg, s);
    case 128: return launch_d<T, D, 128>(which, a, arg, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
hipError_t launch_t(int d, int dv, int which, const BwdArgs& a, int arg, hipStream_t s) {
  switch (d) {
    case 32: return launch_v<T, 32>(dv, which, a, arg, s);
    case 64: return launch_v<T, 64>(dv, which, a, arg, s);
    case 128: return launch_v<T, 128>(dv, which, a, arg, s);
    default: return hipErrorInvalidValue;
  }
}

// d: the key width, dv: the value width
hipError_t launch(int dtype, int d, int dv, int which, const BwdArgs& a, int arg, hipStream_t s) {
  return dtype == kBF16 ? launch_t<bf16>(d, dv, which, a, arg, s)
                        : launch_t<float>(d, dv, which, a, arg, s);
}

}  // namespace

hipError_t launch_fill_f32(float* p, float v, int64_t n, hipStream_t stream) {
  hipLaunchKernelGGL(fill_kernel, dim3(elem_grid(n)), dim3(256), 0, stream, p, v, n);
  return hipGetLastError();
}

hipError_t launch_gemm(int dtype, const GemmArgs& g, hipStream_t stream) {
  const int64_t tiles = (int64_t)((g.M + 63) / 64) * ((g.N + 63) / 64) * g.batches;
  if (tiles <= 0 || tiles > INT32_MAX) return hipErrorInvalidValue;
  if (dtype == kBF16)
    hipLaunchKernelGGL((gemm_kernel<bf16>), dim3((unsigned)tiles), dim3(256), 0, stream, g);
  else
    hipLaunchKernelGGL((gemm_kernel<float>), dim3((unsigned)tiles), dim3(256), 0, stream, g);
  return hipGetLastError();
}

hipError_t launch_bwd_retrieval_rows(int dtype, int d, int dv, const BwdArgs& a, hipStream_t s) {
  return launch(dtype, d, dv, 0, a, 0, s);
}
hipError_t launch_bwd_row_weighted_sum(int dtype, int d, int dv, const BwdArgs& a, bool of_q,
                                       hipStream_t s) {
  return launch(dtype, d, dv, 2, a, of_q ? 1 : 0, s);
}
hipError_t launch_bwd_attention(int dtype, int d, int dv, const BwdArgs& a, hipStream_t s) {
  if (d == dv && attn_bwd_mfma_supported(dtype, d, a.Hq / a.Hkv))
    return launch_attn_bwd_mfma(d, a, s);
  return launch(dtype, d, dv, 3, a, 0, s);  // float, d = 32 or two widths: one wave per row
}
hipError_t launch_bwd_update_rows(int dtype, int d, int dv, const BwdArgs& a, hipStream_t s) {
  return launch(dtype, d, dv, 4, a, 0, s);
}
hipError_t launch_bwd_finish(int dtype, int d, int dv, const BwdArgs& a, hipStream_t s) {
  return launch(dtype, d, dv, 5, a, 0, s);
}
hipError_t launch_bwd_phi_rows(int dtype, int d, int dv, const BwdArgs& a, hipStream_t s) {
  return launch(dtype, d, dv, 6, a, 0, s);
}
hipError_t launch_round_f32(int dtype, void* dst, const float* src, int64_t n, hipStream_t s) {
  if (dtype == kBF16)
    hipLaunchKernelGGL((round_kernel<bf16>), dim3(elem_grid(n)), dim3(256), 0, s,
                       static_cast<bf16*>(dst), src, n);
  else
    hipLaunchKernelGGL((round_kernel<float>), dim3(elem_grid(n)), dim3(256), 0, s,
                       static_cast<float*>(dst), src, n);
  return hipGetLastError();
}

}  // namespace infini

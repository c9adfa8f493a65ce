// The memory scan: the sequential half of the block forward.
//
// "Infini-Attention" (AI Wiki), "How does the compressive memory work?": after
// a segment, M absorbs sigma(K)^T V (additive variant) or
// sigma(K)^T (V - sigma(K) M_{s-1} / (sigma(K) z_{s-1})) (delta rule), and z
// absorbs sum_t sigma(K_t). "Hugging Face Infini-Attention Reproduction
// Analysis", "Infini-Attention Mechanism", step 6: only (M, z) crosses the
// segment boundary.
//
// Design. The value columns of M evolve independently under both rules (the
// delta prediction's denominator sigma(K) z does not involve M), so M is split
// into 32-column slabs and each workgroup owns one (batch, KV head, slab) for
// the whole window, with no communication between workgroups. The slab lives
// in LDS in float; a copy in the element type, stored transposed (M^T), feeds
// the MFMA that forms the delta prediction. Each of the NW waves takes 32
// tokens of a step of 32*NW tokens and accumulates its share of the segment's
// update in MFMA accumulators; the shares are added to the float state in wave
// order at the end of the segment, so results are deterministic. Before each
// segment the workgroup writes the state it starts from (M^T in the element
// type, z in float) for the attention kernel's retrieval.
//
// Per step and wave (32 tokens x 32 value columns):
//   Phi = sigma(K rows)            -> registers (A operand) and Phi^T in LDS
//   den_t = Phi_t . z_{s-1}        -> float, from the unrounded Phi
//   P = Phi M_{s-1}                -> one 32x32 accumulator (delta only)
//   dM += Phi^T V - Phi^T (P/den)  -> d/32 accumulators, two products
// z's column sums are kept per lane in float and reduced across lanes once per
// segment with a reduce-scatter of fixed order.
#include "common.hpp"
#include "kernels.hpp"

namespace infini {

namespace {

// One reduce-scatter step across the lanes that differ in `mask`: the lane
// whose `mask` bit is clear keeps the sums of the first half of its CNT values,
// the other lane those of the second half.
template <int CNT>
__device__ __forceinline__ void reduce_scatter_step(float* a, int mask, bool upper) {
#pragma unroll
  for (int j = 0; j < CNT / 2; ++j) {
    const float send = upper ? a[j] : a[j + CNT / 2];
    const float keep = upper ? a[j + CNT / 2] : a[j];
    a[j] = keep + __shfl_xor(send, mask);
  }
}

// DK: the key width (rows of M, length of z); DV: the value width (columns
// of M, split into 32-column slabs).
template <typename T, int DK, int DV, int RULE, int NW>
__global__ __launch_bounds__(NW * 64) void scan_kernel(ScanArgs a) {
  constexpr int NT = NW * 64;
  constexpr int TOK = 32 * NW;          // tokens per step
  constexpr int NC = DK / 16;           // 16-wide chunks of the key dimension
  constexpr int NDB = DK / 32;          // 32-row blocks of the key dimension
  constexpr int NZ = NC * 8;            // key-dimension entries a lane touches (DK / 2)
  constexpr int MTS = DK + pad16<T>();  // row stride of Mt
  constexpr int PTS = TOK + pad16<T>();  // row stride of PhiT
  constexpr int MSS = 33;               // row stride of Ms (float)
  static_assert(NT >= DK, "one thread per entry of z");

  __shared__ __align__(16) T Mt[32 * MTS];    // M_{s-1}^T of the slab, element type
  __shared__ __align__(16) T PhiT[DK * PTS];  // sigma(K)^T of the current step
  __shared__ float Ms[DK * MSS];              // the slab of M in float, [key][value]
  __shared__ float den_s[TOK];
  __shared__ float zprev[DK];
  __shared__ float zred[NW * DK];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int i = lane & 31, h = lane >> 5;
  const int unit = blockIdx.x % a.units;
  const int slab = blockIdx.x / a.units;
  const int col0 = slab * 32;

  const T* K = static_cast<const T*>(a.k) + (int64_t)unit * a.L * DK;
  const T* V = static_cast<const T*>(a.v) + (int64_t)unit * a.L * DV;
  const float* Min = a.M_in + (int64_t)unit * DK * DV;
  const float* zin = a.z_in + (int64_t)unit * DK;

  for (int idx = tid; idx < DK * 32; idx += NT) {
    const int dk = idx >> 5, c = idx & 31;
    Ms[dk * MSS + c] = Min[dk * DV + col0 + c];
  }
  for (int idx = tid; idx < DK; idx += NT) zprev[idx] = zin[idx];
  __syncthreads();
  for (int idx = tid; idx < 32 * DK; idx += NT) {
    const int r = idx / DK, dk = idx % DK;
    Mt[r * MTS + dk] = from_f32<T>(Ms[dk * MSS + r]);
  }
  __syncthreads();

  for (int sl = 0; sl < a.s_count; ++sl) {
    const int64_t seg_start = (int64_t)(a.s_begin + sl) * a.seg_len;
    const int n_s = (int)min<int64_t>(a.seg_len, a.L - seg_start);

    // The state before this segment, for the retrieval.
    {
      T* sM = static_cast<T*>(a.snapM) + ((int64_t)unit * a.s_count + sl) * DV * DK;
      for (int idx = tid; idx < 32 * (DK / 8); idx += NT) {
        const int r = idx / (DK / 8), c8 = (idx % (DK / 8)) * 8;
        store8<T>(sM + (int64_t)(col0 + r) * DK + c8, load8<T>(Mt + r * MTS + c8));
      }
      if (slab == 0) {
        float* sZ = a.snapZ + ((int64_t)unit * a.s_count + sl) * DK;
        for (int idx = tid; idx < DK; idx += NT) sZ[idx] = zprev[idx];
      }
    }

    frag_t<T> mfr[NC];  // B operand of P = Phi M_{s-1}: column i of M is row i of Mt
    if constexpr (RULE == kRuleDelta) {
#pragma unroll
      for (int c = 0; c < NC; ++c) mfr[c] = load8<T>(Mt + i * MTS + 16 * c + 8 * h);
    }
    f32x16 dM[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) dM[db] = zero16();
    float zp[NZ];
#pragma unroll
    for (int q = 0; q < NZ; ++q) zp[q] = 0.f;

    for (int t0 = 0; t0 < n_s; t0 += TOK) {
      const int tok = t0 + 32 * w + i;
      const bool valid = tok < n_s;
      const T* krow = K + (seg_start + tok) * DK;
      frag_t<T> phf[NC];
      float dpart = 0.f;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        frag_t<T> kv = zero_frag<T>();
        if (valid) kv = load8<T>(krow + 16 * c + 8 * h);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int dk = 16 * c + 8 * h + e;
          const float p = valid ? feature_map(to_f32<T>(kv[e])) : 0.f;
          zp[c * 8 + e] += p;
          dpart += p * zprev[dk];
          phf[c][e] = from_f32<T>(p);
          PhiT[dk * PTS + 32 * w + i] = phf[c][e];
        }
      }
      const float den = dpart + __shfl_xor(dpart, 32);
      if (h == 0) den_s[32 * w + i] = valid ? den : 1.f;
      __syncthreads();

      f32x16 accp;
      if constexpr (RULE == kRuleDelta) {
        accp = zero16();
#pragma unroll
        for (int c = 0; c < NC; ++c) mma32(accp, phf[c], mfr[c]);
      }
      // V and, for the delta rule, the negated prediction -P/den, in the
      // accumulator layout: register r of lane (i, h) is token acc_row(r, h)
      // of the wave's 32 and value column i of the slab. The two stay separate
      // B operands: V is exact in the element type, while V - P/den rounded
      // as one value would lose most of the (small) prediction to rounding,
      // and that loss adds up coherently over the segment's tokens.
      frag_t<T> vf[2], pf[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tr = acc_row(r, h);
        const int tk = t0 + 32 * w + tr;
        T vv = from_f32<T>(0.f);
        if (tk < n_s) vv = V[(seg_start + tk) * DV + col0 + i];
        vf[r >> 3][r & 7] = vv;
        if constexpr (RULE == kRuleDelta)
          pf[r >> 3][r & 7] = from_f32<T>(-accp[r] / den_s[32 * w + tr]);
      }
      // dM += Phi^T V (- Phi^T P/den): the A operand needs, for key row
      // 32db + i, the tokens that the B operands' register order gives (two
      // runs of four).
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const T* prow = PhiT + (32 * db + i) * PTS + 32 * w + 16 * c + 4 * h;
          const frag_t<T> af = load4x2<T>(prow, prow + 8);
          mma32(dM[db], af, vf[c]);
          if constexpr (RULE == kRuleDelta) mma32(dM[db], af, pf[c]);
        }
      }
      __syncthreads();
    }

    // M_s = M_{s-1} + the waves' shares, added in wave order.
    for (int ww = 0; ww < NW; ++ww) {
      if (w == ww) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) Ms[(32 * db + acc_row(r, h)) * MSS + i] += dM[db][r];
      }
      __syncthreads();
    }

    // z_s = z_{s-1} + sum over the segment's tokens: reduce each half-wave's
    // 32 lanes, then the waves in order.
    {
      const bool b16 = i & 16, b8 = i & 8, b4 = i & 4, b2 = i & 2, b1 = i & 1;
      int base, cnt;
      bool write = true;
      if constexpr (NZ == 64) {
        reduce_scatter_step<64>(zp, 16, b16);
        reduce_scatter_step<32>(zp, 8, b8);
        reduce_scatter_step<16>(zp, 4, b4);
        reduce_scatter_step<8>(zp, 2, b2);
        reduce_scatter_step<4>(zp, 1, b1);
        base = b16 * 32 + b8 * 16 + b4 * 8 + b2 * 4 + b1 * 2;
        cnt = 2;
      } else if constexpr (NZ == 32) {
        reduce_scatter_step<32>(zp, 16, b16);
        reduce_scatter_step<16>(zp, 8, b8);
        reduce_scatter_step<8>(zp, 4, b4);
        reduce_scatter_step<4>(zp, 2, b2);
        reduce_scatter_step<2>(zp, 1, b1);
        base = b16 * 16 + b8 * 8 + b4 * 4 + b2 * 2 + b1;
        cnt = 1;
      } else {
        static_assert(NZ == 16, "d must be 32, 64 or 128");
        reduce_scatter_step<16>(zp, 16, b16);
        reduce_scatter_step<8>(zp, 8, b8);
        reduce_scatter_step<4>(zp, 4, b4);
        reduce_scatter_step<2>(zp, 2, b2);
        zp[0] += __shfl_xor(zp[0], 1);
        base = b16 * 8 + b8 * 4 + b4 * 2 + b2;
        cnt = 1;
        write = !b1;
      }
      if (write) {
        for (int j = 0; j < cnt; ++j) {
          const int q = base + j;
          zred[w * DK + 16 * (q >> 3) + 8 * h + (q & 7)] = zp[j];
        }
      }
      __syncthreads();
      if (tid < DK) {
        float s = zprev[tid];
        for (int ww = 0; ww < NW; ++ww) s += zred[ww * DK + tid];
        zprev[tid] = s;
      }
    }
    for (int idx = tid; idx < 32 * DK; idx += NT) {
      const int r = idx / DK, dk = idx % DK;
      Mt[r * MTS + dk] = from_f32<T>(Ms[dk * MSS + r]);
    }
    __syncthreads();
  }

  float* Mout = a.M_out + (int64_t)unit * DK * DV;
  for (int idx = tid; idx < DK * 32; idx += NT) {
    const int dk = idx >> 5, c = idx & 31;
    Mout[dk * DV + col0 + c] = Ms[dk * MSS + c];
  }
  if (slab == 0) {
    float* zout = a.z_out + (int64_t)unit * DK;
    for (int idx = tid; idx < DK; idx += NT) zout[idx] = zprev[idx];
  }
}

template <typename T, int DK, int DV, int RULE>
hipError_t launch_scan_t(const ScanArgs& a, hipStream_t stream) {
  constexpr int NW = 4;
  const dim3 grid((unsigned)(a.units * (DV / 32)));
  hipLaunchKernelGGL((scan_kernel<T, DK, DV, RULE, NW>), grid, dim3(NW * 64), 0, stream, a);
  return hipGetLastError();
}

template <typename T, int DK, int DV>
hipError_t launch_scan_rule(int rule, const ScanArgs& a, hipStream_t stream) {
  return rule == kRuleDelta ? launch_scan_t<T, DK, DV, kRuleDelta>(a, stream)
                            : launch_scan_t<T, DK, DV, kRuleLinear>(a, stream);
}

template <typename T>
hipError_t launch_scan_d(int d, int rule, const ScanArgs& a, hipStream_t stream) {
  switch (d) {
    case 32: return launch_scan_rule<T, 32, 32>(rule, a, stream);
    case 64: return launch_scan_rule<T, 64, 64>(rule, a, stream);
    case 128: return launch_scan_rule<T, 128, 128>(rule, a, stream);
    default: return hipErrorInvalidValue;
  }
}

// d_key != d_value: every ordered pair of distinct widths in {32, 64, 128}
template <typename T, int DK>
hipError_t launch_scan_kv_v(int dv, int rule, const ScanArgs& a, hipStream_t stream) {
  switch (dv) {
    case 32: return DK != 32 ? launch_scan_rule<T, DK, 32>(rule, a, stream) : hipErrorInvalidValue;
    case 64: return DK != 64 ? launch_scan_rule<T, DK, 64>(rule, a, stream) : hipErrorInvalidValue;
    case 128: return DK != 128 ? launch_scan_rule<T, DK, 128>(rule, a, stream) : hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
hipError_t launch_scan_kv_d(int dk, int dv, int rule, const ScanArgs& a, hipStream_t stream) {
  switch (dk) {
    case 32: return launch_scan_kv_v<T, 32>(dv, rule, a, stream);
    case 64: return launch_scan_kv_v<T, 64>(dv, rule, a, stream);
    case 128: return launch_scan_kv_v<T, 128>(dv, rule, a, stream);
    default: return hipErrorInvalidValue;
  }
}

__global__ void copy_f32_kernel(float* dst, const float* src, int64_t n) {
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n;
       idx += (int64_t)gridDim.x * blockDim.x)
    dst[idx] = src[idx];
}

}  // namespace

hipError_t launch_scan(int dtype, int d, int rule, const ScanArgs& a, hipStream_t stream) {
  return dtype == kBF16 ? launch_scan_d<bf16>(d, rule, a, stream)
                        : launch_scan_d<float>(d, rule, a, stream);
}

hipError_t launch_scan_kv(int dtype, int dk, int dv, int rule, const ScanArgs& a,
                          hipStream_t stream) {
  return dtype == kBF16 ? launch_scan_kv_d<bf16>(dk, dv, rule, a, stream)
                        : launch_scan_kv_d<float>(dk, dv, rule, a, stream);
}

namespace {

// One state as the attention reads it: M^T [dv][dk] in the element type and
// z [dk] in float, per unit; thread t of the unit's blocks writes element t of
// M^T (reading M [dk][dv] with stride dv).
template <typename T>
__global__ __launch_bounds__(256) void snapshot_kernel(const float* M, const float* z, T* snapM,
                                                       float* snapZ, int dk, int dv) {
  const int unit = blockIdx.y;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx < dk * dv) {
    const int j = idx / dk, i = idx % dk;  // M^T row j (value column), column i (key row)
    snapM[(int64_t)unit * dk * dv + idx] = static_cast<T>(M[(int64_t)unit * dk * dv + (int64_t)i * dv + j]);
  }
  if (blockIdx.x == 0 && threadIdx.x < dk)
    snapZ[(int64_t)unit * dk + threadIdx.x] = z[(int64_t)unit * dk + threadIdx.x];
}

}  // namespace

hipError_t launch_snapshot(int dtype, int dk, int dv, const float* M, const float* z,
                           void* snapM, float* snapZ, int64_t units, hipStream_t stream) {
  const dim3 grid((unsigned)((dk * dv + 255) / 256), (unsigned)units);
  if (dtype == kBF16)
    hipLaunchKernelGGL(snapshot_kernel<bf16>, grid, dim3(256), 0, stream, M, z,
                       static_cast<bf16*>(snapM), snapZ, dk, dv);
  else
    hipLaunchKernelGGL(snapshot_kernel<float>, grid, dim3(256), 0, stream, M, z,
                       static_cast<float*>(snapM), snapZ, dk, dv);
  return hipGetLastError();
}

hipError_t launch_copy_f32(float* dst, const float* src, int64_t n, hipStream_t stream) {
  const int64_t blocks = (n + 255) / 256;
  const unsigned g = (unsigned)(blocks < 1024 ? (blocks < 1 ? 1 : blocks) : 1024);
  hipLaunchKernelGGL(copy_f32_kernel, dim3(g), dim3(256), 0, stream, dst, src, n);
  return hipGetLastError();
}

}  // namespace infini

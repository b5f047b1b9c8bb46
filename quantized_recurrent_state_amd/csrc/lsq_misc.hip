// fp32-state decode step (the unquantised mode and the FP32-state baseline),
// calibration of an fp32 state into a quantised handle, and the zero fill.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lsq_step_impl.h"

namespace lsq {

Geometry geometry(int bits, int dk) {
  Geometry g{};
  if (bits == 32)
    g.lanes_per_row = 4;                 // interleaved fp32 layout, see step_f32_kernel
  else
    g.lanes_per_row = dk / dev::EPL;     // 32 elements per lane
  g.rows_per_iter = 64 / g.lanes_per_row;
  return g;
}

namespace dev {

// fp32 state.  Four lanes cover a row; lane lc owns the float4 chunks at
// columns 16j + 4lc .. 16j + 4lc + 3 (j = 0 .. DK/16-1), so each load
// instruction reads 64 contiguous bytes of every row the wave touches.
// Arithmetic is Eq. (1) in the same fp32 order as the quantised kernels:
// S' = fl(S * alpha_c), u = S'.k, w = fl(beta fl(v - u)), S = fma(w, k, S').
template <int DK, int DELTA, int DIAG>
__global__ __launch_bounds__(256) void step_f32_kernel(StepArgs a) {
  constexpr int LPR = 4, RPI = 16, NC = DK / 16, EPL = DK / 4;
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wave >= a.total_waves) return;
  const int h = wave / a.waves_per_head;
  const int slice = wave - h * a.waves_per_head;
  const int lr = lane / LPR, lc = lane % LPR;

  float kk[EPL], qq[EPL], aa[DIAG ? EPL : 4];
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const int c = 16 * j + 4 * lc;
    const float4 k4 = *reinterpret_cast<const float4*>(a.k + (size_t)h * DK + c);
    const float4 q4 = *reinterpret_cast<const float4*>(a.q + (size_t)h * DK + c);
    kk[4 * j] = k4.x; kk[4 * j + 1] = k4.y; kk[4 * j + 2] = k4.z; kk[4 * j + 3] = k4.w;
    qq[4 * j] = q4.x; qq[4 * j + 1] = q4.y; qq[4 * j + 2] = q4.z; qq[4 * j + 3] = q4.w;
    if constexpr (DIAG) {
      const float4 a4 = *reinterpret_cast<const float4*>(a.alpha + (size_t)h * DK + c);
      aa[4 * j] = a4.x; aa[4 * j + 1] = a4.y; aa[4 * j + 2] = a4.z; aa[4 * j + 3] = a4.w;
    }
  }
  const float alpha_s = DIAG ? 1.f : a.alpha[h];
  const float beta = a.beta[h];

  for (int it = 0; it < a.nit; ++it) {
    const int r = (slice * a.nit + it) * RPI + lr;
    const bool live = r < a.dv;
    const size_t row = (size_t)h * a.dv + (live ? r : a.dv - 1);
    float* srow = a.ref + row * DK;
    float sp[EPL];
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const float4 x = *reinterpret_cast<const float4*>(srow + 16 * j + 4 * lc);
      sp[4 * j] = x.x; sp[4 * j + 1] = x.y; sp[4 * j + 2] = x.z; sp[4 * j + 3] = x.w;
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) sp[e] = sp[e] * (DIAG ? aa[e] : alpha_s);
    float u = 0.f;
    if constexpr (DELTA) {
      float p = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) p = fmaf(sp[e], kk[e], p);
      u = row_sum<LPR>(p);
    }
    const float w = beta * (a.v[row] - u);
    float po = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      sp[e] = fmaf(w, kk[e], sp[e]);
      po = fmaf(sp[e], qq[e], po);
    }
    const float o = row_sum<LPR>(po);
    if (live) {
#pragma unroll
      for (int j = 0; j < NC; ++j)
        *reinterpret_cast<float4*>(srow + 16 * j + 4 * lc) =
            make_float4(sp[4 * j], sp[4 * j + 1], sp[4 * j + 2], sp[4 * j + 3]);
      if (lc == 0) a.o[row] = o;
    }
  }
}

// Quantise an fp32 state: absmax group scale, round-half-even codes, clamp.
// Same lane layout as the step kernels (32 elements per lane); GPL = 2 for
// 16-element groups (two groups inside a lane).
template <int BITS, int DK, int GPL>
__global__ __launch_bounds__(256) void calibrate_kernel(CalibArgs a) {
  using F = Fmt<BITS>;
  constexpr int LPR = DK / EPL, RPI = 64 / LPR, ROWB = DK * BITS / 8;
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wave >= a.total_waves) return;
  const int h = wave / a.waves_per_head;
  const int slice = wave - h * a.waves_per_head;
  const int lr = lane / LPR, lc = lane % LPR, col0 = lc * EPL;
  const int gl = a.group / EPL, gi = col0 / a.group;
  for (int it = 0; it < a.nit; ++it) {
    const int r = (slice * a.nit + it) * RPI + lr;
    const bool live = r < a.dv;
    const size_t row = (size_t)h * a.dv + (live ? r : a.dv - 1);
    float x[EPL];
    load_f32(x, a.S + row * DK + col0);
    float amax[GPL] = {};
#pragma unroll
    for (int e = 0; e < EPL; ++e)
      amax[GPL == 2 ? e / 16 : 0] = fmaxf(amax[GPL == 2 ? e / 16 : 0], fabsf(x[e]));
    float s[GPL], inv[GPL];
    uint32_t s16[GPL] = {};
#pragma unroll
    for (int g = 0; g < GPL; ++g) {
      s[g] = (GPL == 2 ? amax[g] : group_max(amax[g], gl)) / F::QMAX;
      if (a.sfmt != SFMT_F32) {          // codes are formed with the stored scale
        s16[g] = scale_to16(s[g], a.sfmt);
        s[g] = scale_from16(s16[g], a.sfmt);
      }
      inv[g] = inv_scale(s[g]);
    }
    float t[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e)
      t[e] = __builtin_amdgcn_fmed3f(fmaf(x[e], inv[GPL == 2 ? e / 16 : 0], F::MQ), F::MQ - F::QMAX,
                                     F::MQ + F::QMAX);
    uint32_t X[F::NW];
    pack_offsets<BITS>(t, X);
    if (live) {
      uint8_t* p = a.codes + row * ROWB + lc * (EPL * BITS / 8);
#pragma unroll
      for (int c = 0; c < F::NW / 4; ++c)
        reinterpret_cast<uint4*>(p)[c] = make_uint4(X[4 * c] ^ F::OFF, X[4 * c + 1] ^ F::OFF,
                                                    X[4 * c + 2] ^ F::OFF, X[4 * c + 3] ^ F::OFF);
      if (a.sfmt != SFMT_F32) {
        uint16_t* s16p = reinterpret_cast<uint16_t*>(a.scales) + row * a.ng + gi;
        if constexpr (GPL == 2)
          *reinterpret_cast<uint32_t*>(s16p) = s16[0] | (s16[1] << 16);
        else if ((lc % gl) == 0)
          *s16p = (uint16_t)s16[0];
      } else if constexpr (GPL == 2) {
        *reinterpret_cast<float2*>(a.scales + row * a.ng + gi) = make_float2(s[0], s[1]);
      } else {
        if ((lc % gl) == 0) a.scales[row * a.ng + gi] = s[0];
      }
      if (a.ref) store_f32(a.ref + row * DK + col0, x);
    }
  }
}

__global__ void fill_zero_kernel(uint4* p, size_t n16, uint32_t* tail, size_t ntail) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
  if (blockIdx.x == 0 && threadIdx.x < ntail) tail[threadIdx.x] = 0u;
}

}  // namespace dev

hipError_t launch_step_f32(const StepArgs& a, int dk, int delta, int diag, hipStream_t s) {
  const dim3 grid((a.total_waves + 3) / 4), block(256);
#define LSQ_F32(DK, D, G)                                                               \
  if (dk == DK && delta == D && diag == G) {                                            \
    hipLaunchKernelGGL((dev::step_f32_kernel<DK, D, G>), grid, block, 0, s, a);         \
    return hipGetLastError();                                                           \
  }
  LSQ_F32(128, 0, 0) LSQ_F32(128, 0, 1) LSQ_F32(128, 1, 0) LSQ_F32(128, 1, 1)
  LSQ_F32(64, 0, 0) LSQ_F32(64, 0, 1) LSQ_F32(64, 1, 0) LSQ_F32(64, 1, 1)
#undef LSQ_F32
  return hipErrorInvalidValue;
}

hipError_t launch_calibrate(const CalibArgs& a, int bits, int dk, hipStream_t s) {
  const dim3 grid((a.total_waves + 3) / 4), block(256);
#define LSQ_CAL(B, DK)                                                                  \
  if (bits == B && dk == DK) {                                                          \
    if (a.group < dev::EPL)                                                             \
      hipLaunchKernelGGL((dev::calibrate_kernel<B, DK, 2>), grid, block, 0, s, a);      \
    else                                                                                \
      hipLaunchKernelGGL((dev::calibrate_kernel<B, DK, 1>), grid, block, 0, s, a);      \
    return hipGetLastError();                                                           \
  }
  LSQ_CAL(4, 128) LSQ_CAL(4, 64) LSQ_CAL(8, 128) LSQ_CAL(8, 64)
#undef LSQ_CAL
  return hipErrorInvalidValue;
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
  if (bytes == 0) return hipSuccess;
  const size_t n16 = bytes / 16, ntail = (bytes % 16) / 4;
  uint32_t* tail = reinterpret_cast<uint32_t*>(static_cast<char*>(p) + n16 * 16);
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks == 0) blocks = 1;
  hipLaunchKernelGGL(dev::fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     reinterpret_cast<uint4*>(p), n16, tail, ntail);
  return hipGetLastError();
}


namespace dev {

// S = fl(C s) for every element: one thread per 16 bytes of codes (32 INT4
// or 16 INT8 elements of one row), 16-byte loads and stores.
template <int BITS, int DK>
__global__ __launch_bounds__(256) void dequantize_kernel(DequantArgs a) {
  constexpr int ROWB = DK * BITS / 8, TPR = ROWB / 16, EPT = 16 * 8 / BITS;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= a.rows * TPR) return;
  const int64_t row = t / TPR;
  const int c0 = (int)(t - row * TPR) * EPT;
  const uint4 w4 = *reinterpret_cast<const uint4*>(a.codes + row * ROWB + (c0 * BITS) / 8);
  const uint32_t w[4] = {w4.x, w4.y, w4.z, w4.w};
  float out[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const uint32_t word = w[(e * BITS) / 32], sh = (e * BITS) % 32;
    const int code = BITS == 4 ? ((int)(word << (28 - sh)) >> 28) : ((int)(word << (24 - sh)) >> 24);
    const int64_t si = a.group == 0 ? row / a.dv : row * a.ng + (c0 + e) / a.group;
    float s;
    if (a.sfmt == SFMT_F32)
      s = reinterpret_cast<const float*>(a.scales)[si];
    else
      s = scale_from16(reinterpret_cast<const uint16_t*>(a.scales)[si], a.sfmt);
    out[e] = (float)code * s;
  }
  float4* dst = reinterpret_cast<float4*>(a.S + row * DK + c0);
#pragma unroll
  for (int e = 0; e < EPT / 4; ++e)
    dst[e] = make_float4(out[4 * e], out[4 * e + 1], out[4 * e + 2], out[4 * e + 3]);
}

}  // namespace dev

hipError_t launch_dequantize(const DequantArgs& a, int bits, int dk, hipStream_t s) {
  const int64_t threads = a.rows * (dk * bits / 8 / 16);
  const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
  if (bits == 4 && dk == 128) hipLaunchKernelGGL((dev::dequantize_kernel<4, 128>), grid, block, 0, s, a);
  else if (bits == 4 && dk == 64) hipLaunchKernelGGL((dev::dequantize_kernel<4, 64>), grid, block, 0, s, a);
  else if (bits == 8 && dk == 128) hipLaunchKernelGGL((dev::dequantize_kernel<8, 128>), grid, block, 0, s, a);
  else if (bits == 8 && dk == 64) hipLaunchKernelGGL((dev::dequantize_kernel<8, 64>), grid, block, 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace lsq

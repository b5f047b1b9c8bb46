// Internal interface between the host API (lsq_api.cpp) and the HIP kernels.
// Not installed; the public interface is include/lsq.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lsq {

// Arguments of one decode-step launch (one handle, one step).
struct StepArgs {
  uint8_t* codes;        // [n][dv][dk*bits/8]
  float* scales;         // [n][dv][ng]: fp32, or 16-bit patterns when sfmt != 0
  float* ref;            // [n][dv][dk]  yoked reference (or fp32 state for bits 32)
  const float* q;        // [n][dk]
  const float* k;        // [n][dk]
  const float* v;        // [n][dv]
  const float* alpha;    // [n] or [n][dk]
  const float* beta;     // [n]
  float* o;              // [n][dv]
  float* o_ref;          // [n][dv] or null
  int32_t n_heads;
  int32_t dv;
  int32_t group;
  int32_t ng;            // groups per row = dk / group
  int32_t nit;           // row-iterations per wave
  int32_t waves_per_head;
  int32_t total_waves;
  // dithered rounding: Weyl state of element (r, c) of every head is
  // dither_base + r * dither_row + c * 0x9E3779B9 (mod 2^32)
  uint32_t dither_base;  // (step * dv * dk) * 0x9E3779B9 mod 2^32
  uint32_t dither_row;   // dk * 0x9E3779B9 mod 2^32
  // Low-Rank Bypass (lrb_rank > 0): a [n][r][dv], b [n][2][r][dk]
  float* lrb_a;
  float* lrb_b;
  int32_t lrb_rank;
  int32_t lrb_used;      // slots filled before this step (step mod r)
  int32_t lrb_merge;     // 1 when this step fills the last slot and merges
  int32_t lrb_cin, lrb_cout;  // b copy read / written this step
  int32_t sfmt;          // stored scale format: 0 fp32, 1 binary16, 2 bfloat16
  int32_t head_scale;    // 1: one scale per head (scales [n]), broadcast to every row
  int32_t nt_loads;      // 1: the packed codes exceed the last-level cache by far (non-temporal loads)
};

// Arguments of a calibration launch: quantise an fp32 state into codes/scales.
struct CalibArgs {
  const float* S;        // [n][dv][dk]
  uint8_t* codes;
  float* scales;
  float* ref;            // copy of S for the yoked policy, else null
  int32_t n_heads, dv, group, ng;
  int32_t nit, waves_per_head, total_waves;
  int32_t sfmt;          // stored scale format (as StepArgs)
};

// Arguments of a dequantisation launch: S = fl(C s) of every element.
struct DequantArgs {
  const uint8_t* codes;  // [n][dv][dk*bits/8]
  const void* scales;    // [n][dv][ng] in the stored format, or [n] (one per head)
  float* S;              // [n][dv][dk]
  int64_t rows;          // n * dv
  int32_t dv, group, ng;
  int32_t sfmt;          // stored scale format (as StepArgs)
};

// Arguments of a chunkwise prefill launch (linear write): the handle's packed
// state is advanced over T tokens, one workgroup per head.
struct PrefillArgs {
  uint8_t* codes;        // [n][dv][dk*bits/8]
  float* scales;         // [n][dv][ng]
  const float* k;        // [T][n][dk]
  const float* v;        // [T][n][dv]
  const float* alpha;    // [T][n] or [T][n][dk]
  const float* beta;     // [T][n]
  int32_t n_heads, T, ng, group;
  int32_t sfmt;          // stored scale format (SFMT_*): fp32, binary16 or bfloat16
};

// Launch geometry shared by the host and the kernels.
struct Geometry {
  int32_t lanes_per_row;   // lanes covering one state row
  int32_t rows_per_iter;   // rows one wave covers per iteration (64 / lanes_per_row)
};

Geometry geometry(int bits, int dk);

// Launchers.  Each returns hipErrorInvalidValue when no kernel instance
// matches (the host API checks support before calling).
hipError_t launch_step_q4(const StepArgs& a, int dk, int policy, int rounding, int delta, int diag,
                          hipStream_t s);
hipError_t launch_step_q8(const StepArgs& a, int dk, int policy, int rounding, int delta, int diag,
                          hipStream_t s);
hipError_t launch_step_q4_f16(const StepArgs& a, int dk, int policy, int rounding, int delta,
                              int diag, hipStream_t s);
hipError_t launch_step_q4_bf16(const StepArgs& a, int dk, int policy, int rounding, int delta,
                               int diag, hipStream_t s);
hipError_t launch_step_q8_f16(const StepArgs& a, int dk, int policy, int rounding, int delta,
                              int diag, hipStream_t s);
hipError_t launch_step_q8_bf16(const StepArgs& a, int dk, int policy, int rounding, int delta,
                               int diag, hipStream_t s);
hipError_t launch_step_f32(const StepArgs& a, int dk, int delta, int diag, hipStream_t s);
hipError_t launch_calibrate(const CalibArgs& a, int bits, int dk, hipStream_t s);
hipError_t launch_lrb_step(const StepArgs& a, int bits, int dk, int policy, int rounding,
                           int delta, int diag, hipStream_t s);
hipError_t launch_lrb_step_r8(const StepArgs& a, int bits, int dk, int policy, int rounding,
                              int delta, int diag, hipStream_t s);
hipError_t launch_prefill(const PrefillArgs& a, int bits, int dk, int dv, int policy, int diag,
                          hipStream_t s);
hipError_t launch_bdr_alt(const StepArgs& a, int bits, int dk, int rounding, int delta, int diag,
                          hipStream_t s);
hipError_t launch_head_scale(const StepArgs& a, int bits, int dk, int policy, int rounding,
                             int delta, int diag, hipStream_t s);
hipError_t launch_calibrate_head(const CalibArgs& a, int bits, int dk, hipStream_t s);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);
hipError_t launch_dequantize(const DequantArgs& a, int bits, int dk, hipStream_t s);
// Streaming probe (include/lsq_probe.h): kind 0 read, 1 write, 2 copy.
hipError_t launch_probe(int kind, const void* src, void* dst, size_t bytes, int loads_per_lane,
                        int nontemporal, int workgroups, hipStream_t s);
hipError_t launch_probe_span(const void* src, void* dst, size_t bytes, int span_kib, int nontemporal,
                             hipStream_t s);
// VALU issue probe (include/lsq_probe.h): form 0 fma, 1 med3, 2 mixed.
hipError_t launch_probe_valu(int form, int workgroups, int iters, float* out, hipStream_t s);

}  // namespace lsq

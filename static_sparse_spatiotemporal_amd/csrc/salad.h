// Launchers of the SALAD gate and output kernels (salad_bf16.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace tra {

// Workspace of the gate: one fp32 partial sum per (sample, part of the
// tokens), 256-byte rounded.
size_t salad_gate_workspace_bytes(int64_t B, int64_t N);

// gate[b] = mean_n sigmoid(x[b, n, :] . w + bias); x element (b, n, c) at
// x + b * sx[0] + n * sx[1] + c.
hipError_t launch_salad_gate(const void *x, const int64_t sx[2], const void *w, float bias, int64_t B, int64_t N,
                             int64_t C, float *gate, void *workspace, hipStream_t stream);

// The gate on the library's own scratch array (no allocation, no
// workspace): kGateScratchFloats partial sums, enough for B samples of N
// tokens while B * min(1024, ceil(N / 64)) <= kGateScratchFloats (any N for
// B <= 64).  All calls on one device share the array: calls that overlap in
// time on a device race.
constexpr int64_t kGateScratchFloats = 65536;  // 256 KB per device
bool salad_gate_scratch_fits(int64_t B, int64_t N);
hipError_t launch_salad_gate_scratch(const void *x, const int64_t sx[2], const void *w, float bias, int64_t B,
                                     int64_t N, int64_t C, float *gate, hipStream_t stream);

// out = O_s + gate[b] * (O_l W^T + bias) over the merged-head channels; the
// three tensors are [B, H, N, D] views with element strides s_*[0..2] for
// B, H, N (unit stride in D).
hipError_t launch_salad_combine(const void *os, const int64_t s_os[3], const void *ol, const int64_t s_ol[3],
                                void *out, const int64_t s_out[3], const void *w, const float *bias,
                                const float *gate, int64_t B, int64_t H, int64_t N, int64_t D, hipStream_t stream);

}  // namespace tra

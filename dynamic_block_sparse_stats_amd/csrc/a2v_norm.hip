// a2v_norm.hip -- the A2V norm field a later layer's plan consumes (arXiv 2610.05416;
// nanless digest, guidance section: the audio injection strength of a video position is
// the vector length of its output of the audio-to-video cross-attention, cached from the
// previous layer for the next layer's shape estimation; the first layer has none).
//
// a2v_norm[n] = sqrt(sum_c x[n][c]^2) over the C channels of token n's output row (all
// heads concatenated: one field shared by every head).  One wave per token row: lanes
// stride the row in 16-byte chunks (coalesced), square and sum in float64 (squares of
// the field's far tails, |x| ~ 1e-24, underflow float32; the kernel is HBM-bound, so the
// float64 arithmetic is free), and reduce across the wave.  N * C * b bytes read, 4 N
// written.
#include "prism_internal.h"

namespace prism {

constexpr int kNormWaves = 4;

template <typename T>
__global__ void __launch_bounds__(kNormWaves * 64)
    a2v_norm_kernel(const T *__restrict__ x, long long n_tokens, int channels, long long ld,
                    float *__restrict__ out) {
  constexpr int VPC = 16 / (int)sizeof(T);  // values per 16-byte chunk
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * kNormWaves + (threadIdx.x >> 6);
  if (row >= n_tokens) return;
  const T *p = x + row * ld;
  const int chunks = channels / VPC;
  double acc = 0.0;
  for (int c = lane; c < chunks; c += 64) {
    const u32x4 w = *reinterpret_cast<const u32x4 *>(p + (size_t)c * VPC);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (sizeof(T) == 2) {
        const double lo = __uint_as_float(w[e] << 16), hi = __uint_as_float(w[e] & 0xffff0000u);
        acc = fma(lo, lo, acc);
        acc = fma(hi, hi, acc);
      } else {
        const double f = __uint_as_float(w[e]);
        acc = fma(f, f, acc);
      }
    }
  }
  // channels not a multiple of the chunk width: the tail element by element
  for (int c = chunks * VPC + lane; c < channels; c += 64) {
    double f;
    if constexpr (sizeof(T) == 2)
      f = bf16_to_f32(reinterpret_cast<const uint16_t *>(p)[c]);
    else
      f = reinterpret_cast<const float *>(p)[c];
    acc = fma(f, f, acc);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (lane == 0) out[row] = (float)sqrt(acc);
}

hipError_t launch_a2v_norm(const void *x, long long n_tokens, int channels, long long ld,
                           int dtype, float *out, hipStream_t s) {
  const long long blocks = (n_tokens + kNormWaves - 1) / kNormWaves;
  if (dtype == PRISM_BF16)
    hipLaunchKernelGGL(a2v_norm_kernel<uint16_t>, dim3((unsigned)blocks), dim3(kNormWaves * 64),
                       0, s, (const uint16_t *)x, n_tokens, channels, ld, out);
  else
    hipLaunchKernelGGL(a2v_norm_kernel<float>, dim3((unsigned)blocks), dim3(kNormWaves * 64), 0,
                       s, (const float *)x, n_tokens, channels, ld, out);
  return hipGetLastError();
}

}  // namespace prism

// One kernel per operator, intermediates materialized in HBM: the baseline
// the stitched kernels are measured against ([AStitch] "What people did
// before": skipping fusion yields a kernel storm whose intermediates round-trip
// through DRAM; [sass2mlir] "What graphs deliberately don't do": replaying the
// same chain as a graph removes launch cost but not the round trips).
// Broadcast operands are folded into the consumer's indexing, as a fusing
// compiler would do for the cheap one-to-one part.
#include "dev.hpp"
#include "kernels.hpp"

namespace cf {

namespace {
constexpr int kB = 256;

__device__ __forceinline__ float apply(int op, float x, float c) {
  switch (op) {
    case 0: return x - c;
    case 1: return x / c;
    case 2: return x * c;
    default: return x + c;
  }
}

inline int grid_for(int64_t n) {
  int64_t g = (n + kB - 1) / kB;
  return (int)(g < 65536 ? (g < 1 ? 1 : g) : 65536);
}
}  // namespace

// Row reduction, one wave per row (rows narrower than 2048) or one workgroup
// per row: the rigid row-to-block mapping of a generic reduce kernel.
__global__ __launch_bounds__(kB) void u_k_rowreduce_wave(const float* x, float* out, int64_t rows, int64_t cols, int is_max) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (kB / 64) + (threadIdx.x >> 6);
  if (row >= rows) return;
  const float* xr = x + row * cols;
  float v = is_max ? -INFINITY : 0.0f;
  for (int64_t j = lane; j < cols; j += 64) v = is_max ? fmaxf(v, xr[j]) : v + xr[j];
  v = is_max ? group_reduce<OpMax, 64>(v) : group_reduce<OpSum, 64>(v);
  if (lane == 0) out[row] = v;
}

__global__ __launch_bounds__(kB) void u_k_rowreduce_block(const float* x, float* out, int64_t, int64_t cols, int is_max) {
  __shared__ float s[kB / 64];
  const int64_t row = blockIdx.x;
  const float* xr = x + row * cols;
  float v = is_max ? -INFINITY : 0.0f;
  for (int64_t j = threadIdx.x; j < cols; j += kB) v = is_max ? fmaxf(v, xr[j]) : v + xr[j];
  v = is_max ? group_reduce<OpMax, 64>(v) : group_reduce<OpSum, 64>(v);
  if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    float r = s[0];
    for (int k = 1; k < kB / 64; ++k) r = is_max ? fmaxf(r, s[k]) : r + s[k];
    out[row] = r;
  }
}

__global__ __launch_bounds__(kB) void u_k_bcast_col(const float* x, const float* c, float* y, int64_t rows, int64_t cols, int op) {
  const int64_t n = rows * cols;
  for (int64_t i = (int64_t)blockIdx.x * kB + threadIdx.x; i < n; i += (int64_t)gridDim.x * kB)
    y[i] = apply(op, x[i], c[i / cols]);
}

__global__ __launch_bounds__(kB) void u_k_bcast_row(const float* x, const float* r, float* y, int64_t rows, int64_t cols, int op) {
  const int64_t n = rows * cols;
  for (int64_t i = (int64_t)blockIdx.x * kB + threadIdx.x; i < n; i += (int64_t)gridDim.x * kB)
    y[i] = apply(op, x[i], r[i % cols]);
}

__global__ __launch_bounds__(kB) void u_k_map(const float* x, float* y, int64_t n, int op, float p, float q) {
  for (int64_t i = (int64_t)blockIdx.x * kB + threadIdx.x; i < n; i += (int64_t)gridDim.x * kB) {
    const float v = x[i];
    float r;
    switch (op) {
      case 0: r = expf(v); break;
      case 1: r = v * v; break;
      case 2: r = powf(v, p); break;
      case 3: r = rsqrtf(v * q + p); break;
      case 5: r = fmaxf(v, 0.0f); break;
      case 6: r = 0.5f * v * (1.0f + tanhf(0.7978845608028654f * (v + 0.044715f * v * v * v))); break;
      case 7: r = v / (1.0f + expf(-v)); break;
      case 8: r = 1.0f / sqrtf(v); break;
      default: r = v * p; break;
    }
    y[i] = r;
  }
}

__global__ __launch_bounds__(kB) void u_k_add_bf16(const float* x, const uint16_t* r, float* y, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * kB + threadIdx.x; i < n; i += (int64_t)gridDim.x * kB)
    y[i] = x[i] + __uint_as_float((uint32_t)r[i] << 16);
}

__global__ __launch_bounds__(kB) void u_k_cast_bf16(const float* x, uint16_t* y, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * kB + threadIdx.x; i < n; i += (int64_t)gridDim.x * kB)
    y[i] = (uint16_t)bf16_rne(x[i]);
}

// 16-byte fills and copies for cache eviction and counter calibration.
__global__ __launch_bounds__(kB) void u_k_fill(float* p, int64_t n, float v) {
  const int64_t n4 = n / 4;
  for (int64_t i = (int64_t)blockIdx.x * kB + threadIdx.x; i < n4; i += (int64_t)gridDim.x * kB)
    st4(p + 4 * i, make_float4(v, v, v, v));
  for (int64_t i = 4 * n4 + (int64_t)blockIdx.x * kB + threadIdx.x; i < n; i += (int64_t)gridDim.x * kB) p[i] = v;
}

__global__ __launch_bounds__(kB) void u_k_copy(const float* s, float* d, int64_t n) {
  const int64_t n4 = n / 4;
  for (int64_t i = (int64_t)blockIdx.x * kB + threadIdx.x; i < n4; i += (int64_t)gridDim.x * kB)
    st4(d + 4 * i, ld4(s + 4 * i));
  for (int64_t i = 4 * n4 + (int64_t)blockIdx.x * kB + threadIdx.x; i < n; i += (int64_t)gridDim.x * kB) d[i] = s[i];
}

hipError_t u_rowreduce(const float* x, float* out, int64_t rows, int64_t cols, int is_max, hipStream_t st) {
  if (cols >= 2048) {
    hipLaunchKernelGGL(u_k_rowreduce_block, dim3((unsigned)rows), dim3(kB), 0, st, x, out, rows, cols, is_max);
  } else {
    hipLaunchKernelGGL(u_k_rowreduce_wave, dim3((unsigned)((rows + 3) / 4)), dim3(kB), 0, st, x, out, rows, cols, is_max);
  }
  return hipGetLastError();
}

hipError_t u_bcast_col(const float* x, const float* c, float* y, int64_t rows, int64_t cols, int op, hipStream_t st) {
  hipLaunchKernelGGL(u_k_bcast_col, dim3(grid_for(rows * cols)), dim3(kB), 0, st, x, c, y, rows, cols, op);
  return hipGetLastError();
}

hipError_t u_bcast_row(const float* x, const float* r, float* y, int64_t rows, int64_t cols, int op, hipStream_t st) {
  hipLaunchKernelGGL(u_k_bcast_row, dim3(grid_for(rows * cols)), dim3(kB), 0, st, x, r, y, rows, cols, op);
  return hipGetLastError();
}

hipError_t u_map(const float* x, float* y, int64_t n, int op, float p, float q, hipStream_t st) {
  hipLaunchKernelGGL(u_k_map, dim3(grid_for(n)), dim3(kB), 0, st, x, y, n, op, p, q);
  return hipGetLastError();
}

hipError_t u_add_bf16(const float* x, const uint16_t* r, float* y, int64_t n, hipStream_t st) {
  hipLaunchKernelGGL(u_k_add_bf16, dim3(grid_for(n)), dim3(kB), 0, st, x, r, y, n);
  return hipGetLastError();
}

hipError_t u_cast_bf16(const float* x, uint16_t* y, int64_t n, hipStream_t st) {
  hipLaunchKernelGGL(u_k_cast_bf16, dim3(grid_for(n)), dim3(kB), 0, st, x, y, n);
  return hipGetLastError();
}

hipError_t u_fill(float* p, int64_t n, float v, hipStream_t st) {
  hipLaunchKernelGGL(u_k_fill, dim3(grid_for((n + 3) / 4)), dim3(kB), 0, st, p, n, v);
  return hipGetLastError();
}

hipError_t u_copy(const float* s, float* d, int64_t n, hipStream_t st) {
  hipLaunchKernelGGL(u_k_copy, dim3(grid_for((n + 3) / 4)), dim3(kB), 0, st, s, d, n);
  return hipGetLastError();
}

}  // namespace cf

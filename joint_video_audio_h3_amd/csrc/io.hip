// Patch projections into the packed residual stream (gfx950).
//
//   x[r][c] = b[c] + sum_k in[r][k] * W[c][k]      in fp32 [rows][P], W fp32 [D][P]
//
// The video (96-wide) and audio (32-wide) latent patches enter the stream
// through float32 projections that keep float32 weights, inputs and
// accumulation (H3-metal digest, "Specialized projection kernels"), written
// straight into the stream's rows (minimax-h3-mlx README, "Architecture": the
// packed sequence and its two input patch projections).
//
// The contraction runs on the fp32 matrix cores (v_mfma_f32_32x32x2_f32).  The
// two k slots of each MFMA take the two halves of the patch: lane l (row l%32,
// half l/32) holds in[row][half*P/2 + s] for every step s, so its operand is a
// run of P/2 contiguous floats (float4 loads) and P/2 MFMAs cover all P inputs.
// A wavefront owns 32 rows and walks NCT 32-wide column tiles, loading each
// tile's weights (P/2 floats per lane, L2-resident) while the previous tile's
// MFMAs run.  HBM traffic per row: 4*P bytes read, 4*D bytes written.
#include "h3_device.h"
#include "launch.h"

namespace h3 {

constexpr int PE_NCT = 4;   // 32-wide column tiles per wavefront

template <int P>
__global__ __launch_bounds__(256) void patch_embed_kernel(PatchArgs a) {
  constexpr int H = P / 2, V4 = H / 4;
  static_assert(P % 8 == 0 && P <= 128, "patch width");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 31, hl = lane >> 5;
  const int row0 = (blockIdx.x * 4 + wave) * 32;
  if (row0 >= a.rows) return;
  const int col_base = blockIdx.y * (32 * PE_NCT);

  float av[H];
  {
    const int r = min(row0 + lr, a.rows - 1);
    const float4* src = reinterpret_cast<const float4*>(a.in + (size_t)r * P + hl * H);
#pragma unroll
    for (int i = 0; i < V4; ++i) {
      const float4 t = src[i];
      av[4 * i] = t.x; av[4 * i + 1] = t.y; av[4 * i + 2] = t.z; av[4 * i + 3] = t.w;
    }
  }
  auto load_w = [&](int ct, float (&bv)[H]) __attribute__((always_inline)) {
    const int c = min(col_base + ct * 32 + lr, a.D - 1);
    const float4* src = reinterpret_cast<const float4*>(a.W + (size_t)c * P + hl * H);
#pragma unroll
    for (int i = 0; i < V4; ++i) {
      const float4 t = src[i];
      bv[4 * i] = t.x; bv[4 * i + 1] = t.y; bv[4 * i + 2] = t.z; bv[4 * i + 3] = t.w;
    }
  };
  float bw[2][H];
  load_w(0, bw[0]);
#pragma unroll
  for (int ct = 0; ct < PE_NCT; ++ct) {
    const int col0 = col_base + ct * 32;
    if (col0 >= a.D) break;
    if (ct + 1 < PE_NCT) load_w(ct + 1, bw[(ct + 1) & 1]);
    f32x16 acc = f32x16{};
#pragma unroll
    for (int s = 0; s < H; ++s)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av[s], bw[ct & 1][s], acc, 0, 0, 0);
    const int col = col0 + lr;
    if (col < a.D) {
      const float b = a.bias ? a.bias[col] : 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = row0 + 8 * (v / 4) + 4 * hl + (v % 4);
        if (r < a.rows) a.out[(size_t)r * a.D + col] = acc[v] + b;
      }
    }
  }
}

// One Euler pass of a latent: z += dt * v (rectified flow; minimax-h3-mlx
// README, "Layout": rectified-flow Euler with exponential sigma shift).
// float4 pieces; HBM traffic 12 bytes per element.
__global__ __launch_bounds__(256) void euler_kernel(float* z, const float* v, float dt, int64_t n) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i + 3 < n) {
    float4 a = *reinterpret_cast<const float4*>(z + i);
    const float4 b = *reinterpret_cast<const float4*>(v + i);
    a.x += dt * b.x;
    a.y += dt * b.y;
    a.z += dt * b.z;
    a.w += dt * b.w;
    *reinterpret_cast<float4*>(z + i) = a;
  } else {
    for (int64_t j = i; j < n; ++j) z[j] += dt * v[j];
  }
}

hipError_t launch_euler(float* z, const float* v, float dt, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  euler_kernel<<<dim3((unsigned)((n + 1023) / 1024)), 256, 0, s>>>(z, v, dt, n);
  return hipGetLastError();
}

// An Euler pass along a velocity extrapolated from two fresh ones:
// z += dt * (v1 + c * (v1 - v0)) = a * v1 + b * v0 with a = dt * (1 + c),
// b = -dt * c (H3-metal digest, "Sampler and DiT controls": skipped velocities
// are extrapolated on each modality's schedule).  16 bytes per element.
__global__ __launch_bounds__(256) void euler2_kernel(float* z, const float* v1, const float* v0, float a,
                                                     float b, int64_t n) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i + 3 < n) {
    float4 zz = *reinterpret_cast<const float4*>(z + i);
    const float4 p = *reinterpret_cast<const float4*>(v1 + i);
    const float4 q = *reinterpret_cast<const float4*>(v0 + i);
    zz.x += a * p.x + b * q.x;
    zz.y += a * p.y + b * q.y;
    zz.z += a * p.z + b * q.z;
    zz.w += a * p.w + b * q.w;
    *reinterpret_cast<float4*>(z + i) = zz;
  } else {
    for (int64_t j = i; j < n; ++j) z[j] += a * v1[j] + b * v0[j];
  }
}

hipError_t launch_euler2(float* z, const float* v1, const float* v0, float a, float b, int64_t n,
                         hipStream_t s) {
  if (n <= 0) return hipSuccess;
  euler2_kernel<<<dim3((unsigned)((n + 1023) / 1024)), 256, 0, s>>>(z, v1, v0, a, b, n);
  return hipGetLastError();
}

// Count the modality tags outside [0, n_tags) (the optional argument check).
__global__ __launch_bounds__(256) void count_bad_tags_kernel(const int32_t* tag, int64_t n, int n_tags,
                                                             unsigned int* bad) {
  unsigned int c = 0;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    c += (tag[i] < 0 || tag[i] >= n_tags) ? 1u : 0u;
  if (c) atomicAdd(bad, c);
}

// The check's counter lives in the library's static device memory (one per
// device, allocated with the code object), so the check allocates nothing.
static __device__ __align__(256) unsigned int g_bad_tags;

hipError_t bad_tags_counter(unsigned int** ptr) {
  static unsigned int* addr[64] = {nullptr};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  if (!addr[dev]) {
    void* p = nullptr;
    if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_bad_tags))) != hipSuccess) return e;
    addr[dev] = static_cast<unsigned int*>(p);
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_count_bad_tags(const int32_t* tag, int64_t n, int n_tags, unsigned int* bad, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  count_bad_tags_kernel<<<dim3((unsigned)(blocks < 1024 ? blocks : 1024)), 256, 0, s>>>(tag, n, n_tags, bad);
  return hipGetLastError();
}

hipError_t launch_patch_embed(const PatchArgs& a, hipStream_t s) {
  const dim3 grid((a.rows + 127) / 128, (a.D + 32 * PE_NCT - 1) / (32 * PE_NCT));
  switch (a.P) {
    case 32: patch_embed_kernel<32><<<grid, 256, 0, s>>>(a); break;
    case 64: patch_embed_kernel<64><<<grid, 256, 0, s>>>(a); break;
    case 96: patch_embed_kernel<96><<<grid, 256, 0, s>>>(a); break;
    case 128: patch_embed_kernel<128><<<grid, 256, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace h3

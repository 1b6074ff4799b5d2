// AdaLN norm-modulate and the rotary angle table (gfx950).
//
// adaln_kernel: one wavefront per packed row.  The fp32 row stays in registers
// (D/256 float4 per lane), mean and biased variance are two exact passes over
// those registers with wavefront butterfly sums, and the row's (shift, scale)
// pair is gathered from the per-tag modulation table:
//   h = LN(x) * (1 + scale[tag]) + shift[tag]      -> bf16
// (minimax-h3-mlx README, "AdaLN: measure, do not reason": x*(1+scale)+shift
// for the norms; "AdaLN precompute": the table replaces the projection.)
// HBM traffic per row: 4*D bytes read + 2*D bytes written.
//
// quant_groups_kernel / quant_rows_kernel: the int8 codes and scales of the
// W8A8 trunk's bf16 activations (one scale per group of G elements along K,
// or per row).
//
// rope_kernel: cos/sin of pos[r][axis] * theta^(-2j/d_axis) for every channel
// pair, evaluated in double precision once per forward (3D MM-RoPE,
// minimax-h3-mlx README, "Architecture").
#include "h3_device.h"
#include "launch.h"

namespace h3 {

// Per-row symmetric int8 codes (W8A8 activations), in float32 exactly as
// specified: amax = max|v|, inv = 127 / amax, q = clamp(rint(v * inv), +-127),
// scale = amax / 127 (IEEE divisions, rint ties to even; amax = 0 gives 0, 0).
__device__ __forceinline__ uint32_t quant4(float a, float b, float c, float d, float inv) {
  auto one = [&](float v) -> uint32_t {
    const float t = fminf(fmaxf(__builtin_rintf(v * inv), -127.0f), 127.0f);
    return (uint32_t)((int)t & 0xff);
  };
  return one(a) | (one(b) << 8) | (one(c) << 16) | (one(d) << 24);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}

template <int VPL>  // float4 vectors per lane: ceil(D / 256)
__global__ __launch_bounds__(256) void adaln_kernel(AdalnArgs a) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.n) return;
  const int nv = a.D >> 2;
  const float4* xr = reinterpret_cast<const float4*>(a.x + (size_t)row * a.D);
  const int t = a.tag ? a.tag[row] : 0;   // no tags: one (shift, scale) pair for every row
  const u16x4* sh = reinterpret_cast<const u16x4*>(a.table + ((size_t)t * 6 + a.k_shift) * a.D);
  const u16x4* sc = reinterpret_cast<const u16x4*>(a.table + ((size_t)t * 6 + a.k_scale) * a.D);
  float4 v[VPL];
  u16x4 s4v[VPL], c4v[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int j = lane + 64 * i;
    if (j < nv) {
      v[i] = xr[j];
    } else {
      v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  // the row's (shift, scale) entries (L2 hits: n_tags rows) are in flight
  // while the row is reduced, rather than fetched after the reductions
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int j = lane + 64 * i;
    if (j < nv) {
      s4v[i] = sh[j];
      c4v[i] = sc[j];
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < VPL; ++i) s += (v[i].x + v[i].y) + (v[i].z + v[i].w);
  const float mean = wave_sum(s) / (float)a.D;
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int j = lane + 64 * i;
    if (j < nv) {
      const float dx = v[i].x - mean, dy = v[i].y - mean, dz = v[i].z - mean, dw = v[i].w - mean;
      q += (dx * dx + dy * dy) + (dz * dz + dw * dw);
    }
  }
  const float var = wave_sum(q) / (float)a.D;
  const float rstd = 1.0f / sqrtf(var + a.eps);
  uint2* hr = reinterpret_cast<uint2*>(a.h + (size_t)row * a.D);
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int j = lane + 64 * i;
    if (j < nv) {
      const u16x4 s4 = s4v[i], c4 = c4v[i];
      const float o0 = (v[i].x - mean) * rstd * (1.0f + bf2f(c4[0])) + bf2f(s4[0]);
      const float o1 = (v[i].y - mean) * rstd * (1.0f + bf2f(c4[1])) + bf2f(s4[1]);
      const float o2 = (v[i].z - mean) * rstd * (1.0f + bf2f(c4[2])) + bf2f(s4[2]);
      const float o3 = (v[i].w - mean) * rstd * (1.0f + bf2f(c4[3])) + bf2f(s4[3]);
      hr[j] = make_uint2(pack2bf(o0, o1), pack2bf(o2, o3));
    }
  }
}

// Group-scaled int8 codes of a bf16 matrix [n][K] (W8A8 activations; mlx-h3
// README, "Generate": group-scaled W8A8 with groups of 64, 256, 448 or 896
// along K).  For every row and group of G consecutive elements: amax over the
// group, codes q = clamp(rint(v * (127 / amax)), +-127), scale amax / 127,
// every step in IEEE float32 (amax = 0 gives codes 0 and scale 0).  A group is
// P = G/8 pieces of 16 bytes; a wavefront takes 64/P groups of one row when
// P <= 32 (P lanes each, one piece per lane), else one group (its pieces spread
// over the 64 lanes), so the group maximum is a butterfly over the group's own
// lanes.  Scales are stored group-major, s[g][row] with row stride ld (the
// padded row count); rows n .. ld-1 get scale 0.  HBM traffic per row: 2*K
// bytes read, K + 4*K/G written.
template <int G>
__global__ __launch_bounds__(256) void quant_groups_kernel(QuantArgs a) {
  constexpr int P = G / 8;                       // 16-byte pieces per group
  constexpr int SEG = P <= 32 ? 64 / P : 1;      // groups per wavefront
  constexpr int LPG = P <= 32 ? P : 64;          // lanes per group
  constexpr int PPL = (P + LPG - 1) / LPG;       // pieces per lane
  static_assert(G % 8 == 0 && (P > 32 || 64 % P == 0), "groups tile the wavefront");
  const int lane = threadIdx.x & 63;
  const int ng = a.K / G;
  const int wpr = (ng + SEG - 1) / SEG;          // wavefronts per row
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t row = wid / wpr;
  if (row >= a.ld) return;
  const int g = (int)(wid % wpr) * SEG + lane / LPG;
  const int sl = lane % LPG;                     // lane within the group
  const bool live = g < ng;
  if (row >= a.n) {                              // padded rows: scale 0
    if (live && sl == 0) a.s[(size_t)g * a.ld + row] = 0.f;
    return;
  }
  const size_t base = (size_t)row * a.K + (size_t)g * G;
  uint4 v[PPL];
  float amax = 0.f;
  auto lo = [](uint32_t w) { return __uint_as_float(w << 16); };
  auto hi = [](uint32_t w) { return __uint_as_float(w & 0xffff0000u); };
#pragma unroll
  for (int t = 0; t < PPL; ++t) {
    const int pi = sl + LPG * t;
    v[t] = (live && pi < P) ? *reinterpret_cast<const uint4*>(a.in + base + 8 * pi) : make_uint4(0, 0, 0, 0);
    const uint32_t w[4] = {v[t].x, v[t].y, v[t].z, v[t].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) amax = fmaxf(amax, fmaxf(fabsf(lo(w[e])), fabsf(hi(w[e]))));
  }
#pragma unroll
  for (int m = LPG / 2; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
  if (!live) return;
  const float inv = amax > 0.f ? 127.0f / amax : 0.f;
#pragma unroll
  for (int t = 0; t < PPL; ++t) {
    const int pi = sl + LPG * t;
    if (pi < P)
      *reinterpret_cast<uint2*>(a.q + base + 8 * pi) =
          make_uint2(quant4(lo(v[t].x), hi(v[t].x), lo(v[t].y), hi(v[t].y), inv),
                     quant4(lo(v[t].z), hi(v[t].z), lo(v[t].w), hi(v[t].w), inv));
  }
  if (sl == 0) a.s[(size_t)g * a.ld + row] = amax > 0.f ? amax / 127.0f : 0.f;
}

// One scale per row (FC2's per-row form; H3-metal digest, "4. Choose a
// speed/quality preset").  One wavefront per row: the bf16 row stays in
// registers (8 values per 16-byte piece), its absolute maximum is a wavefront
// reduction, then the codes go out 8 bytes per piece; rows n .. ld-1 get scale
// 0.  HBM traffic per row: 2*K bytes read, K + 4 written.
template <int VPL>  // 16-byte pieces per lane: ceil(K / 512)
__global__ __launch_bounds__(256) void quant_rows_kernel(QuantArgs a) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.ld) return;
  if (row >= a.n) {
    if (lane == 0) a.s[row] = 0.f;
    return;
  }
  const int nv = a.K >> 3;
  const uint4* src = reinterpret_cast<const uint4*>(a.in + (size_t)row * a.K);
  uint4 v[VPL];
  float amax = 0.f;
  auto lo = [](uint32_t w) { return __uint_as_float(w << 16); };
  auto hi = [](uint32_t w) { return __uint_as_float(w & 0xffff0000u); };
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int j = lane + 64 * i;
    v[i] = j < nv ? src[j] : make_uint4(0, 0, 0, 0);
    const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
    for (int t = 0; t < 4; ++t) amax = fmaxf(amax, fmaxf(fabsf(lo(w[t])), fabsf(hi(w[t]))));
  }
  amax = wave_max(amax);
  const float inv = amax > 0.f ? 127.0f / amax : 0.f;
  uint2* dst = reinterpret_cast<uint2*>(a.q + (size_t)row * a.K);
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int j = lane + 64 * i;
    if (j < nv)
      dst[j] = make_uint2(quant4(lo(v[i].x), hi(v[i].x), lo(v[i].y), hi(v[i].y), inv),
                          quant4(lo(v[i].z), hi(v[i].z), lo(v[i].w), hi(v[i].w), inv));
  }
  if (lane == 0) a.s[row] = amax > 0.f ? amax / 127.0f : 0.f;
}

#define H3_ADALN_CASE(V) \
  case V: adaln_kernel<V><<<grid, 256, 0, s>>>(a); break;

hipError_t launch_adaln(const AdalnArgs& a, hipStream_t s) {
  const int vpl = (a.D / 4 + 63) / 64;
  const dim3 grid((a.n + 3) / 4);
  switch (vpl) {
    H3_ADALN_CASE(1) H3_ADALN_CASE(2) H3_ADALN_CASE(3) H3_ADALN_CASE(4)
    H3_ADALN_CASE(5) H3_ADALN_CASE(6) H3_ADALN_CASE(7) H3_ADALN_CASE(8)
    H3_ADALN_CASE(9) H3_ADALN_CASE(10) H3_ADALN_CASE(11) H3_ADALN_CASE(12)
    H3_ADALN_CASE(13) H3_ADALN_CASE(14) H3_ADALN_CASE(15) H3_ADALN_CASE(16)
    H3_ADALN_CASE(17) H3_ADALN_CASE(18) H3_ADALN_CASE(19) H3_ADALN_CASE(20)
    H3_ADALN_CASE(21) H3_ADALN_CASE(22) H3_ADALN_CASE(23) H3_ADALN_CASE(24)
    H3_ADALN_CASE(25) H3_ADALN_CASE(26) H3_ADALN_CASE(27) H3_ADALN_CASE(28)
    H3_ADALN_CASE(29) H3_ADALN_CASE(30) H3_ADALN_CASE(31) H3_ADALN_CASE(32)
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

#define H3_QUANT_CASE(V) \
  case V: quant_rows_kernel<V><<<grid, 256, 0, s>>>(a); break;

template <int G>
static hipError_t launch_groups(const QuantArgs& a, hipStream_t s) {
  constexpr int P = G / 8, SEG = P <= 32 ? 64 / P : 1;
  const int64_t waves = (int64_t)a.ld * (((a.K / G) + SEG - 1) / SEG);
  quant_groups_kernel<G><<<dim3((unsigned)((waves + 3) / 4)), 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_quant(const QuantArgs& a, hipStream_t s) {
  if (a.K % 8 != 0 || a.group <= 0 || a.K % a.group != 0 || a.ld < a.n) return hipErrorInvalidValue;
  if (a.group != a.K) {
    switch (a.group) {
      case 64: return launch_groups<64>(a, s);
      case 256: return launch_groups<256>(a, s);
      case 448: return launch_groups<448>(a, s);
      case 896: return launch_groups<896>(a, s);
      default: return hipErrorInvalidValue;
    }
  }
  const int vpl = (a.K / 8 + 63) / 64;
  const dim3 grid((a.ld + 3) / 4);
  switch (vpl) {
    H3_QUANT_CASE(1) H3_QUANT_CASE(2) H3_QUANT_CASE(3) H3_QUANT_CASE(4)
    H3_QUANT_CASE(5) H3_QUANT_CASE(6) H3_QUANT_CASE(7) H3_QUANT_CASE(8)
    H3_QUANT_CASE(9) H3_QUANT_CASE(10) H3_QUANT_CASE(11) H3_QUANT_CASE(12)
    H3_QUANT_CASE(13) H3_QUANT_CASE(14) H3_QUANT_CASE(15) H3_QUANT_CASE(16)
    H3_QUANT_CASE(17) H3_QUANT_CASE(18) H3_QUANT_CASE(19) H3_QUANT_CASE(20)
    H3_QUANT_CASE(21) H3_QUANT_CASE(22) H3_QUANT_CASE(23) H3_QUANT_CASE(24)
    H3_QUANT_CASE(25) H3_QUANT_CASE(26) H3_QUANT_CASE(27) H3_QUANT_CASE(28)
    H3_QUANT_CASE(29) H3_QUANT_CASE(30) H3_QUANT_CASE(31) H3_QUANT_CASE(32)
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void rope_kernel(RopeArgs a) {
  const int half = a.d / 2;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)a.n_pad * half) return;
  const int row = (int)(idx / half);
  const int p = (int)(idx % half);
  int axis, j, width;
  if (p < a.split0 / 2) {
    axis = 0; j = p; width = a.split0;
  } else if (p < (a.split0 + a.split1) / 2) {
    axis = 1; j = p - a.split0 / 2; width = a.split1;
  } else {
    axis = 2; j = p - (a.split0 + a.split1) / 2; width = a.split2;
  }
  const double pos = row < a.n ? (double)a.pos[(size_t)row * 3 + axis] : 0.0;
  const double ang = pos * pow(a.theta, -2.0 * (double)j / (double)width);
  double sn, cn;
  sincos(ang, &sn, &cn);
  reinterpret_cast<float2*>(a.cs)[idx] = make_float2((float)cn, (float)sn);
}

hipError_t launch_rope_table(const RopeArgs& a, hipStream_t s) {
  const int64_t total = (int64_t)a.n_pad * (a.d / 2);
  rope_kernel<<<dim3((unsigned)((total + 255) / 256)), 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace h3

// bf16 MFMA GEMM for the four linear layers of the H3 block, with the
// element-wise work of each layer fused into its epilogue (gfx950).
//
//   C[M][n_out] = A[M][K] . B[n_out][K]^T       (A = activations, B = weights,
//                                                 both K-contiguous)
//
// Tiling: BM x BN block tile, BK = 64, WM x WN wavefronts, each owning a
// (BM/WM) x (BN/WN) sub-tile computed with v_mfma_f32_32x32x16_bf16 (fp32
// accumulators).  A and B tiles are staged through registers into a
// double-buffered LDS ring (row stride 72 bf16 = 144 B, which keeps the
// 16-byte fragment reads of a 16-lane group on distinct banks).  One barrier
// per K step.  Block ids are remapped so that each XCD (blocks are dealt
// round-robin to the 8 XCDs) walks a contiguous run of the grouped tile order,
// and consecutive tiles on an XCD share the same weight tile in its L2.
//
// MFMA 32x32 accumulator layout: lane l, register v holds
//   row = 8*(v/4) + 4*(l/32) + (v%4),   col = l%32.
//
// Epilogues (page titles and sections):
//  EPI_RESID  x[r][c] += gate[tag_r][c] * (acc + bias[c])  -- residual gate of
//             the attention and MLP branches (minimax-h3-mlx README, "AdaLN:
//             measure, do not reason": x + gate * f(x)).  fp32 in place.
//  EPI_SWIGLU weights rows are [gate; value]; each wave's N range is half gate
//             rows and half the matching value rows, so silu(g)*v is formed in
//             registers and only the F-wide activation is written
//             (minimax-h3-mlx README, "Validation": fc2(silu(gate) * value);
//             H3-metal digest, "Metal 4 and TensorOps paths": paired gate/up
//             tiles apply SwiGLU before writing).
//  EPI_QKV    each wave's N range is exactly one head_dim section of the
//             per-head interleaved [q|k|v] projection; q and k get RMSNorm
//             over the section (half-wave butterfly), the gain, and the rotary
//             turn (pair partner is the neighbouring lane), q is pre-scaled by
//             log2(e)/sqrt(d) for the exp2 softmax, and the results are
//             scattered head-major: q, k [H][n_pad][d], v transposed
//             [H][d][n_pad] (H3-metal digest, "Checkpoint layout and media
//             pipeline" and "Metal 4 and TensorOps paths": fused
//             QK-normalisation/RoPE, Q/K/V routed straight to head-major
//             attention inputs).
//  INT8 (wfmt 1): B is int8 with one bf16 scale per 32 K elements; each
//             16-byte chunk of codes is dequantised to bf16(q*s) on its way
//             into LDS, so the MFMA loop is the same as the bf16 path's.
#include "h3_device.h"
#include "launch.h"

namespace h3 {

constexpr int BK = 64;
constexpr int LDK = BK + 8;

template <int BM, int BN, int WM, int WN, int EPI, int WF, int SEC>
__global__ __launch_bounds__(WM* WN * 64) void gemm_kernel(GemmArgs p) {
  constexpr int NT = WM * WN * 64;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int A_CH = BM * 8 / NT;
  constexpr int B_CH = WF == 0 ? BN * 8 / NT : BN * 4 / NT;
  static_assert(A_CH * NT == BM * 8 && B_CH > 0, "tile/thread mismatch");
  static_assert(EPI != EPI_QKV || TN == SEC, "QKV wave tile must be one head section");
  static_assert(EPI != EPI_SWIGLU || FN % 2 == 0, "SwiGLU needs paired gate/value tiles");

  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (BM + BN) * LDK];
  __shared__ int s_tag[EPI == EPI_RESID ? BM : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // ---- tile coordinates: XCD-aware remap, then grouped order along M
  const int tiles_m = (EPI == EPI_QKV) ? p.n_pad / BM : (p.M + BM - 1) / BM;
  const int tiles_n = (p.n_out + BN - 1) / BN;
  const int total = tiles_m * tiles_n;
  int pid;
  {
    const int raw = blockIdx.x;
    const int per = total / 8, rem = total % 8;
    const int xcd = raw % 8, local = raw / 8;
    pid = xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
  }
  constexpr int GROUP_M = 8;
  const int in_group = GROUP_M * tiles_n;
  const int first_m = (pid / in_group) * GROUP_M;
  const int gsz = min(tiles_m - first_m, GROUP_M);
  const int tm = first_m + (pid % in_group) % gsz;
  const int tn = (pid % in_group) / gsz;
  const int m0 = tm * BM;
  const int n0 = tn * BN;

  if (EPI == EPI_RESID) {
    for (int i = tid; i < BM; i += NT) s_tag[i] = p.tag[min(m0 + i, p.M - 1)];
  }

  // ---- per-thread global source rows
  const int K = p.K;
  const uint16_t* a_src[A_CH];
#pragma unroll
  for (int i = 0; i < A_CH; ++i) {
    const int c = tid + i * NT;
    const int r = min(m0 + c / 8, p.M - 1);
    a_src[i] = p.A + (size_t)r * K + (c % 8) * 8;
  }
  constexpr int B_PER_ROW = WF == 0 ? 8 : 4;
  const uint8_t* b_src[B_CH];
  const uint16_t* s_src[B_CH];
#pragma unroll
  for (int i = 0; i < B_CH; ++i) {
    const int c = tid + i * NT;
    const int r = c / B_PER_ROW;
    int brow;
    if (EPI == EPI_SWIGLU) {
      const int w = r / TN, cc = r % TN, half = TN / 2;
      const int base = tn * (BN / 2) + w * half;
      brow = cc < half ? base + cc : p.ffn + base + cc - half;
    } else {
      brow = min(n0 + r, p.n_out - 1);
    }
    if (WF == 0) {
      b_src[i] = reinterpret_cast<const uint8_t*>(p.B) + ((size_t)brow * K + (c % 8) * 8) * 2;
    } else {
      b_src[i] = reinterpret_cast<const uint8_t*>(p.B) + (size_t)brow * K + (c % 4) * 16;
      s_src[i] = p.Bs + (size_t)brow * (K / 32) + (c % 4) / 2;
    }
  }

  uint4 ra[A_CH];
  uint4 rb[B_CH];
  uint16_t rs[WF == 1 ? B_CH : 1];

  auto gload = [&](int kt) {
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < A_CH; ++i) ra[i] = *reinterpret_cast<const uint4*>(a_src[i] + k0);
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      if (WF == 0) {
        rb[i] = *reinterpret_cast<const uint4*>(b_src[i] + (size_t)k0 * 2);
      } else {
        rb[i] = *reinterpret_cast<const uint4*>(b_src[i] + k0);
        rs[i] = s_src[i][k0 / 32];
      }
    }
  };
  auto sstore = [&](int buf) {
    uint16_t* As = smem + buf * (BM + BN) * LDK;
    uint16_t* Bsm = As + BM * LDK;
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int c = tid + i * NT;
      *reinterpret_cast<uint4*>(As + (c / 8) * LDK + (c % 8) * 8) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const int c = tid + i * NT;
      if (WF == 0) {
        *reinterpret_cast<uint4*>(Bsm + (c / 8) * LDK + (c % 8) * 8) = rb[i];
      } else {
        const float s = bf2f(rs[i]);
        const uint32_t w[4] = {rb[i].x, rb[i].y, rb[i].z, rb[i].w};
        uint32_t o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t word = w[e / 2];
          const int sh = (e % 2) * 16;
          const float lo = (float)(int8_t)((word >> sh) & 0xff) * s;
          const float hi = (float)(int8_t)((word >> (sh + 8)) & 0xff) * s;
          o[e] = pack2bf(lo, hi);
        }
        uint16_t* dst = Bsm + (c / 4) * LDK + (c % 4) * 16;
        *reinterpret_cast<uint4*>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
        *reinterpret_cast<uint4*>(dst + 8) = make_uint4(o[4], o[5], o[6], o[7]);
      }
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

  const int KT = K / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  const int lrow = lane & 31, lk = (lane >> 5) * 8;
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) gload(kt + 1);
    const uint16_t* As = smem + cur * (BM + BN) * LDK + (wm * TM + lrow) * LDK + lk;
    const uint16_t* Bsm = smem + cur * (BM + BN) * LDK + BM * LDK + (wn * TN + lrow) * LDK + lk;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8 af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = *reinterpret_cast<const bf16x8*>(As + i * 32 * LDK + kk * 16);
#pragma unroll
      for (int j = 0; j < FN; ++j) bfr[j] = *reinterpret_cast<const bf16x8*>(Bsm + j * 32 * LDK + kk * 16);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma32(af[i], bfr[j], acc[i][j]);
    }
    if (kt + 1 < KT) sstore(cur ^ 1);
    __syncthreads();
  }

  // ---------------------------------------------------------------- epilogues
  const int hl = lane >> 5;     // half-wave: rows 4..7 of each group of 8
  const int lc = lane & 31;     // column within a 32-wide MFMA tile
  const int row_base = m0 + wm * TM;

  if constexpr (EPI == EPI_RESID) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = n0 + wn * TN + j * 32 + lc;
      if (col >= p.n_out) continue;
      const float b = p.bias ? bf2f(p.bias[col]) : 0.f;
#pragma unroll
      for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int rl = wm * TM + i * 32 + 8 * (v / 4) + 4 * hl + (v % 4);
          const int row = m0 + rl;
          if (row < p.M) {
            const float g = bf2f(p.gate_tab[(size_t)s_tag[rl] * p.tag_stride + col]);
            float* xp = p.x + (size_t)row * p.ldx + col;
            *xp = *xp + g * (acc[i][j][v] + b);
          }
        }
      }
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
    for (int j = 0; j < FN / 2; ++j) {
      const int oc = tn * (BN / 2) + wn * (TN / 2) + j * 32 + lc;
      const float bg = p.bias ? bf2f(p.bias[oc]) : 0.f;
      const float bv = p.bias ? bf2f(p.bias[p.ffn + oc]) : 0.f;
#pragma unroll
      for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = row_base + i * 32 + 8 * (v / 4) + 4 * hl + (v % 4);
          if (row < p.M) {
            const float g = acc[i][j][v] + bg;
            const float u = acc[i][j + FN / 2][v] + bv;
            const float a = g / (1.0f + __expf(-g)) * u;
            p.out[(size_t)row * p.ffn + oc] = f2bf(a);
          }
        }
      }
    }
  } else {  // EPI_QKV
    const int sec = (n0 + wn * TN) / SEC;
    if (sec >= 3 * p.heads) return;
    const int kind = sec % 3, head = sec / 3;
    const uint16_t* gam = kind == 0 ? p.gq : p.gk;
    float bias_c[FN], gain_c[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int c = j * 32 + lc;
      bias_c[j] = p.bias ? bf2f(p.bias[sec * SEC + c]) : 0.f;
      gain_c[j] = (kind < 2 && gam) ? bf2f(gam[c]) : 1.f;
    }
    const float2* cs = reinterpret_cast<const float2*>(p.cs);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      float u[FN][16];
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) u[j][v] = acc[i][j][v] + bias_c[j];
      if (kind < 2) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          float ss = 0.f;
#pragma unroll
          for (int j = 0; j < FN; ++j) ss += u[j][v] * u[j][v];
          ss = half_sum(ss);
          const float r = 1.0f / sqrtf(ss / (float)SEC + p.qk_eps);
          const int row = row_base + i * 32 + 8 * (v / 4) + 4 * hl + (v % 4);
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const float t = u[j][v] * r * gain_c[j];
            const float partner = __shfl_xor(t, 1, 64);
            const int c = j * 32 + lc;
            const float2 sc = cs[(size_t)row * (SEC / 2) + c / 2];
            float o = (c & 1) ? partner * sc.y + t * sc.x : t * sc.x - partner * sc.y;
            if (kind == 0) o *= p.q_scale;
            u[j][v] = o;
          }
        }
      }
      uint16_t* dst = kind == 0 ? p.q : p.k;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = row_base + i * 32 + 8 * (v / 4) + 4 * hl + (v % 4);
        const bool valid = row < p.M;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int c = j * 32 + lc;
          const uint16_t val = valid ? f2bf(u[j][v]) : (uint16_t)0;
          if (kind < 2) {
            dst[((size_t)head * p.n_pad + row) * SEC + c] = val;
          } else {
            p.vt[((size_t)head * SEC + c) * p.n_pad + row] = val;
          }
        }
      }
    }
  }
}

template <int BM, int BN, int WM, int WN, int EPI, int WF, int SEC>
static hipError_t run(const GemmArgs& a, hipStream_t s) {
  const int tiles_m = (EPI == EPI_QKV) ? a.n_pad / BM : (a.M + BM - 1) / BM;
  const int tiles_n = (a.n_out + BN - 1) / BN;
  gemm_kernel<BM, BN, WM, WN, EPI, WF, SEC><<<dim3(tiles_m * tiles_n), WM * WN * 64, 0, s>>>(a);
  return hipGetLastError();
}

template <int WF>
static hipError_t dispatch(int epi, const GemmArgs& a, hipStream_t s) {
  switch (epi) {
    case EPI_RESID:
      return run<256, 256, 2, 2, EPI_RESID, WF, 0>(a, s);
    case EPI_SWIGLU:
      return run<256, 256, 2, 2, EPI_SWIGLU, WF, 0>(a, s);
    case EPI_QKV:
      if (a.head_dim == 128) return run<256, 256, 2, 2, EPI_QKV, WF, 128>(a, s);
      if (a.head_dim == 96) return run<256, 192, 2, 2, EPI_QKV, WF, 96>(a, s);
      return hipErrorInvalidValue;
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm(int epi, int wfmt, const GemmArgs& a, hipStream_t s) {
  return wfmt == 0 ? dispatch<0>(epi, a, s) : dispatch<1>(epi, a, s);
}

}  // namespace h3

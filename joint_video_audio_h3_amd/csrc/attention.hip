// Flash-style full attention over the packed sequence (gfx950, MFMA bf16).
//
//   o = softmax(q k^T / sqrt(d)) v   per head, over all n keys, no mask
// (minimax-h3-mlx README, "Architecture": full self-attention over the one
// packed sequence; "Performance": flash-style, the score matrix is never
// materialised).
//
// Work split: a block of 4 wavefronts takes 128 queries of one head; each
// wavefront owns 32 queries and walks all keys in tiles of 64, with K and V^T
// tiles double-buffered in LDS.  Scores are computed transposed,
//   S^T[key][query] = K . Q^T       (MFMA A = K rows, B = Q fragment)
// so that every lane holds one query (lane % 32) and 16 of its keys per
// 32-key sub-tile: the running max and sum need only the two half-waves
// combined.  The K rows are read from LDS in a permuted order chosen so that
// accumulator register v of lane l holds key 16*(v/8) + 8*(l/32) + v%8; the
// probabilities then already sit where the PV product wants its B operand:
//   O^T[dd][query] += V^T[dd][key] . P^T[key][query]
// V^T comes straight from the QKV epilogue (keys contiguous), so both MFMA
// operands are 16-byte LDS reads.  q arrives pre-scaled by log2(e)/sqrt(d),
// so the softmax uses exp2 directly; the running max and row sums are fp32.
// Keys at or beyond n are masked in the last tile; padded rows of q/k/v^T are
// zeros written by the QKV epilogue, so every operand is finite.
#include "h3_device.h"
#include "launch.h"

namespace h3 {

constexpr int ATT_BQ = 128;  // queries per block
constexpr int ATT_BKV = 64;  // keys per tile

template <int HD>
__global__ __launch_bounds__(256) void attn_kernel(AttnArgs p) {
  constexpr int KLD = HD + 8;        // LDS row stride of the K tile (bf16)
  constexpr int VLD = ATT_BKV + 8;   // LDS row stride of the V^T tile
  constexpr int DS = HD / 16;        // MFMA k-steps over head_dim
  constexpr int DT = HD / 32;        // 32-row tiles of head_dim in O^T
  constexpr int K_CH = ATT_BKV * HD / 8 / 256;   // 16-byte chunks per thread
  constexpr int V_CH = HD * ATT_BKV / 8 / 256;
  static_assert(K_CH * 256 * 8 == ATT_BKV * HD && V_CH * 256 * 8 == HD * ATT_BKV, "chunking");
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][ATT_BKV * KLD];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][HD * VLD];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int head = blockIdx.y;
  const int q0 = blockIdx.x * ATT_BQ + wave * 32;
  const int hl = lane >> 5, lq = lane & 31;
  const size_t hoff = (size_t)head * p.n_pad * HD;

  // Q fragments (B operand): query q0+lq, channels ds*16 + 8*hl .. +7
  bf16x8 qf[DS];
  {
    const uint16_t* qp = p.q + hoff + (size_t)(q0 + lq) * HD + 8 * hl;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) qf[ds] = *reinterpret_cast<const bf16x8*>(qp + ds * 16);
  }

  const uint16_t* kbase = p.k + hoff;
  const uint16_t* vbase = p.vt + (size_t)head * HD * p.n_pad;
  uint4 rk[K_CH], rv[V_CH];
  auto gload = [&](int kt) {
    const int key0 = kt * ATT_BKV;
#pragma unroll
    for (int i = 0; i < K_CH; ++i) {
      const int c = tid + i * 256;
      const int r = c / (HD / 8), cc = c % (HD / 8);
      rk[i] = *reinterpret_cast<const uint4*>(kbase + (size_t)(key0 + r) * HD + cc * 8);
    }
#pragma unroll
    for (int i = 0; i < V_CH; ++i) {
      const int c = tid + i * 256;
      const int r = c / (ATT_BKV / 8), cc = c % (ATT_BKV / 8);
      rv[i] = *reinterpret_cast<const uint4*>(vbase + (size_t)r * p.n_pad + key0 + cc * 8);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < K_CH; ++i) {
      const int c = tid + i * 256;
      const int r = c / (HD / 8), cc = c % (HD / 8);
      *reinterpret_cast<uint4*>(&Ks[buf][r * KLD + cc * 8]) = rk[i];
    }
#pragma unroll
    for (int i = 0; i < V_CH; ++i) {
      const int c = tid + i * 256;
      const int r = c / (ATT_BKV / 8), cc = c % (ATT_BKV / 8);
      *reinterpret_cast<uint4*>(&Vs[buf][r * VLD + cc * 8]) = rv[i];
    }
  };

  // K row read by this lane for MFMA row index lq: key = 8h + 4g + c within
  // each 16, for lq = 8g' + 4h + c  (g' = 2*(g/2)... see header comment)
  const int g8 = lq >> 3, h4 = (lq >> 2) & 1, c4 = lq & 3;
  const int krow = 16 * (g8 >> 1) + 8 * h4 + 4 * (g8 & 1) + c4;

  f32x16 oacc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) oacc[t] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  const int NKT = (p.n + ATT_BKV - 1) / ATT_BKV;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < NKT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < NKT) gload(kt + 1);

    f32x16 sacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const uint16_t* kp = &Ks[cur][(ks * 32 + krow) * KLD + 8 * hl];
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(kp + ds * 16);
        sacc[ks] = mfma32(a, qf[ds], sacc[ks]);
      }
    }
    // mask keys >= n (only the last tile can hold them)
    if ((kt + 1) * ATT_BKV > p.n) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = kt * ATT_BKV + ks * 32 + 16 * (v / 8) + 8 * hl + (v % 8);
          if (key >= p.n) sacc[ks][v] = -INFINITY;
        }
    }
    float mx = m_run;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[ks][v]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float alpha = __builtin_amdgcn_exp2f(m_run - mx);
    m_run = mx;
    float rs = 0.f;
    bf16x8 pf[4];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float e = __builtin_amdgcn_exp2f(sacc[ks][v] - mx);
        rs += e;
        pf[ks * 2 + v / 8][v % 8] = (__bf16)e;
      }
    }
    l_run = l_run * alpha + rs;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int v = 0; v < 16; ++v) oacc[t][v] *= alpha;
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      const uint16_t* vp = &Vs[cur][(t * 32 + lq) * VLD + 8 * hl];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(vp + s * 16);
        oacc[t] = mfma32(a, pf[s], oacc[t]);
      }
    }
    if (kt + 1 < NKT) sstore(cur ^ 1);
    __syncthreads();
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.0f / l_tot;
  const int qrow = q0 + lq;
  if (qrow < p.n) {
    uint16_t* op = p.o + (size_t)qrow * p.heads * HD + head * HD;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dd = t * 32 + 8 * g + 4 * hl;
        const uint2 w = make_uint2(pack2bf(oacc[t][4 * g] * inv, oacc[t][4 * g + 1] * inv),
                                   pack2bf(oacc[t][4 * g + 2] * inv, oacc[t][4 * g + 3] * inv));
        *reinterpret_cast<uint2*>(op + dd) = w;
      }
  }
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  const dim3 grid((a.n + ATT_BQ - 1) / ATT_BQ, a.heads);
  if (a.head_dim == 128) {
    attn_kernel<128><<<grid, 256, 0, s>>>(a);
  } else if (a.head_dim == 96) {
    attn_kernel<96><<<grid, 256, 0, s>>>(a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace h3

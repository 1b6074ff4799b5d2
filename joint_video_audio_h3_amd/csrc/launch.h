// Host-side launchers of the gfx950 kernels (one per step of the block).
// Shapes are validated by the C-ABI layer before any of these is called.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace h3 {

struct RopeArgs {
  const float* pos;     // [n][3]
  float* cs;            // [n_pad][d/2][2]
  int n, n_pad, d;
  int split0, split1, split2;
  double theta;
};
hipError_t launch_rope_table(const RopeArgs& a, hipStream_t s);

struct AdalnArgs {
  const float* x;        // [n][D]
  const int32_t* tag;    // [n], or null: every row uses table entry 0
  const uint16_t* table; // [T][6][D]
  uint16_t* h;           // [n][D] bf16 output
  int n, D, k_shift, k_scale;
  float eps;
};
hipError_t launch_adaln(const AdalnArgs& a, hipStream_t s);

// Symmetric int8 quantization of a bf16 matrix [n][K] (W8A8 activations), one
// scale per group of `group` consecutive K elements (group == K: per row).
struct QuantArgs {
  const uint16_t* in;    // [n][K] bf16
  int8_t* q;             // [n][K]
  float* s;              // [K/group][ld] group-major; rows n..ld-1 set to 0
  int n, K, group, ld;
};
hipError_t launch_quant(const QuantArgs& a, hipStream_t s);

enum Epi { EPI_RESID = 0, EPI_SWIGLU = 1, EPI_QKV = 2, EPI_STORE = 3 };

struct GemmArgs {
  const uint16_t* A;      // [M][K] bf16 (int8 codes for W8A8)
  const void* B;          // [Nw][K] bf16 or int8
  const uint16_t* Bs;     // bf16 weight scales: [Nw][K/32] (INT8 g32), [K/group][Nw]
                          // (W8A8) or [Nw] (W8A8 per row)
  const float* sa;        // fp32 scales of int8 A (W8A8): [K/group][sa_ld], or [M] per row
  int group;              // W8A8: K elements per scale group (0: one scale per row)
  int sa_ld;              // W8A8: row stride of sa (the padded row count)
  const uint16_t* bias;   // [Nw] or null
  int M, K;
  int n_out;              // GEMM output columns (= B rows used)
  // EPI_RESID: x[M][ldx] += gate_tab[tag*6*D + col] * (acc + bias)
  // EPI_STORE: x[M][ldx]  = acc + bias
  float* x; int ldx;
  const uint16_t* gate_tab; const int32_t* tag; int tag_stride;
  // EPI_SWIGLU: out[M][ffn] = silu(gate) * value, gate rows [0,ffn), value rows [ffn, 2ffn)
  uint16_t* out; int ffn;
  // EPI_QKV
  uint16_t *q, *k, *vt; int n_pad, heads, head_dim;
  const uint16_t *gq, *gk; const float* cs; float qk_eps, q_scale;
};
hipError_t launch_gemm(int epi, int wfmt, const GemmArgs& a, hipStream_t s);

// bf16 weights [rows][K] = RNE_bf16(q * s) from INT8 group-32 codes and scales
struct DequantArgs {
  const int8_t* q;       // [rows][K]
  const uint16_t* s;     // [rows][K/32] bf16
  uint16_t* out;         // [rows][K] bf16
  int rows, K;
};
hipError_t launch_dequant_w8(const DequantArgs& a, hipStream_t s);

struct AttnArgs {
  const uint16_t *q, *k, *vt;  // [H][n_pad][d], [H][n_pad][d], [H][d][n_pad]
  uint16_t* o;                 // [n][H*d]
  int n, n_pad, heads, head_dim;
  // block-sparse: per (head, query tile) CSR lists of selected key tiles of
  // `tile` rows (64 or 128); tile_idx == null means full attention
  const int32_t* tile_off;     // [heads * ceil(n / tile) + 1]
  const int32_t* tile_idx;
  int tile;
};
hipError_t launch_attention(const AttnArgs& a, hipStream_t s);

struct PatchArgs {
  const float* in;       // [rows][P] fp32 latent patches
  const float* W;        // [D][P] fp32
  const float* bias;     // [D] fp32 or null
  float* out;            // [rows][D] fp32 (rows of the packed stream)
  int rows, P, D;
};
hipError_t launch_patch_embed(const PatchArgs& a, hipStream_t s);

// z[0..n) += dt * v[0..n)  (one Euler pass of a latent)
hipError_t launch_euler(float* z, const float* v, float dt, int64_t n, hipStream_t s);
// z[0..n) += a * v1[0..n) + b * v0[0..n)  (an Euler pass along an extrapolated velocity)
hipError_t launch_euler2(float* z, const float* v1, const float* v0, float a, float b, int64_t n,
                         hipStream_t s);

// Unfused epilogues (H3_UNFUSED=1): plain kernels over a GEMM's fp32 output.
struct UnfusedQkvArgs {
  const float* u;        // [n][3 * heads * head_dim]: per head [q | k | v] sections (acc + bias)
  const uint16_t *gq, *gk;   // bf16 [head_dim] norm gains, or null (1)
  const float* cs;       // [n_pad][head_dim / 2][2] rotary (cos, sin)
  uint16_t *q, *k, *vt;  // [H][n_pad][d], [H][n_pad][d], [H][d][n_pad]; pad rows written as 0
  int n, n_pad, heads, head_dim;
  float eps, q_scale;
};
hipError_t launch_unfused_qkv(const UnfusedQkvArgs& a, hipStream_t s);
// out[n][F] = silu(z[:, :F]) * z[:, F:] (bf16) from z fp32 [n][2F]
hipError_t launch_unfused_swiglu(const float* z, int64_t n, int F, uint16_t* out, hipStream_t s);
// x[n][D] += gate[tag[r] * tag_stride + c] * y[r][c]
hipError_t launch_unfused_resid(const float* y, int64_t n, int D, const uint16_t* gate, const int32_t* tag,
                                int tag_stride, float* x, hipStream_t s);

// device address of the tag check's counter on the current device
hipError_t bad_tags_counter(unsigned int** ptr);
// device address of the library's static scratch array (H3_NOALLOC_SCRATCH_BYTES)
// on the current device, looked up once per device
hipError_t noalloc_scratch(void** ptr);
// *bad += number of tag[0..n) outside [0, n_tags)
hipError_t launch_count_bad_tags(const int32_t* tag, int64_t n, int n_tags, unsigned int* bad, hipStream_t s);

}  // namespace h3

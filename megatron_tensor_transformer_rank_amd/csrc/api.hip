// C ABI of libtpmlp.so: host-side validation, workspace layout and dispatch
// of one tensor-parallel rank's MLP shard onto the gfx950 kernels.
//
// Every check runs before the first launch, so an invalid call enqueues
// nothing.  No exception crosses the ABI; nothing is printed.
#include <atomic>
#include <climits>
#include <cstring>
#include <initializer_list>
#include <new>

#include "common.h"
#include "gemm.h"
#include "gemv.h"
#include "norm.h"
#include "reduce.h"
#include "skinny.h"
#include "tp_mlp.h"

using namespace tpmlp;

namespace {

constexpr int MAX_DEVICES = 64;
// CUs per device, queried once per device (0 = not yet known).
std::atomic<int> g_num_cu[MAX_DEVICES];

int num_cu_current() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return 256;
  int n = g_num_cu[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  g_num_cu[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Scratch of the entry points that allocate nothing (tp_mlp_fwd_shard_noalloc):
// a fixed array in device memory, one copy per GPU, held until the process
// ends.  In host code `scratch` only names the symbol; its device address on
// the current GPU is looked up once per device and kept in g_scratch.
constexpr size_t STATIC_SCRATCH_BYTES = (size_t)64 << 20;
static __device__ __align__(256) uint8_t scratch[STATIC_SCRATCH_BYTES];
std::atomic<void*> g_scratch[MAX_DEVICES];

// The current device's copy of `scratch`, or NULL when the device or the
// symbol cannot be queried.
void* static_scratch_current() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return nullptr;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
  g_scratch[dev].store(p, std::memory_order_release);
  return p;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool opt_aligned(const void* p) { return p == nullptr || aligned16(p); }
bool req(const void* p) { return p != nullptr && aligned16(p); }
// A required buffer of `bytes` bytes; when it is empty (no tokens or rows)
// it may be NULL, as the storage of an empty tensor is.
bool req_n(const void* p, uint64_t bytes) { return bytes == 0 ? opt_aligned(p) : req(p); }

struct Dims {
  int64_t N, h, Fi;
  int act, g;
};

bool check_shape(const tp_mlp_shape* s, Dims& d) {
  if (s == nullptr) return false;
  if (s->n_tokens < 0 || s->hidden < 8 || s->ffn < 1) return false;
  if (s->t < 1 || s->t > MAX_T) return false;  // t > MAX_T: see shape_status
  if (s->rank < 0 || s->rank >= s->t) return false;
  if (s->act != TP_MLP_ACT_RELU && s->act != TP_MLP_ACT_GELU && s->act != TP_MLP_ACT_SWIGLU) return false;
  if (s->ffn % s->t != 0) return false;
  d.N = s->n_tokens;
  d.h = s->hidden;
  d.Fi = s->ffn / s->t;
  d.act = s->act;
  d.g = s->act == TP_MLP_ACT_SWIGLU ? 2 : 1;
  if (d.h % 8 != 0 || d.Fi % 8 != 0 || d.Fi < 8) return false;
  // GEMM extents are int32 inside the kernels
  const int64_t lim = 0x7fffffffLL;
  if (d.N > lim || d.h > lim || 2 * d.Fi > lim) return false;
  return true;
}

// Every GEMM operand is addressed through a 32-bit buffer resource.
bool fits_buffers(const Dims& d) {
  const uint64_t cap = GEMM_MAX_OPERAND_BYTES / 2;  // elements
  const uint64_t N = (uint64_t)d.N, h = (uint64_t)d.h, Fi = (uint64_t)d.Fi, g = (uint64_t)d.g;
  return N * h <= cap && N * g * Fi <= cap && h * Fi <= cap;
}

// INVALID_ARG for a malformed shape, UNSUPPORTED for a well-formed one with
// t above the supported maximum.
tp_mlp_status shape_status(const tp_mlp_shape* s, Dims& d) {
  if (check_shape(s, d)) return fits_buffers(d) ? TP_MLP_OK : TP_MLP_ERR_UNSUPPORTED;
  if (s != nullptr && s->t > MAX_T && s->rank >= 0 && s->rank < s->t) return TP_MLP_ERR_UNSUPPORTED;
  return TP_MLP_ERR_INVALID_ARG;
}

struct DecodeLayout {
  GemvPlan up, down;
  size_t off_part_up, off_part_down, off_cnt, total;
};

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// Small-batch path (2 <= N <= SK_MAX_N): split-K plans aiming at one block
// per CU of a 256-CU MI355X.  A constant, not the device's CU count, so the
// workspace size depends on the shape only.
constexpr int SKINNY_TARGET_BLOCKS = 256;

struct SkinnyLayout {
  SkinnyPlan up, down;
  size_t off_part_up, off_part_down, total;
};

bool small_batch(const Dims& d) { return d.N >= 2 && d.N <= SK_MAX_N; }

SkinnyLayout skinny_layout(const Dims& d) {
  SkinnyLayout L;
  L.up = skinny_plan((int)d.N, (int)d.h, (int)d.Fi, d.g, SKINNY_TARGET_BLOCKS, INT_MAX);
  L.down = skinny_plan((int)d.N, (int)d.Fi, (int)d.h, 1, SKINNY_TARGET_BLOCKS, INT_MAX);
  size_t off = 0;
  L.off_part_up = off;
  off = round256(off + L.up.part_floats * sizeof(float));
  L.off_part_down = off;
  off = round256(off + L.down.part_floats * sizeof(float));
  L.total = off;
  return L;
}

DecodeLayout decode_layout(const Dims& d) {
  DecodeLayout L;
  L.up = gemv_plan((int)d.h, (int)d.Fi, d.g, DECODE_UP_BLOCKS);
  L.down = gemv_plan((int)d.Fi, (int)d.h, 1, DECODE_DOWN_BLOCKS);
  size_t off = 0;
  L.off_part_up = off;
  off = round256(off + L.up.part_floats * sizeof(float));
  L.off_part_down = off;
  off = round256(off + L.down.part_floats * sizeof(float));
  L.off_cnt = off;  // one counter per column strip of the down-projection
  off = round256(off + (size_t)L.down.strips * sizeof(int));
  L.total = off;
  return L;
}

tp_mlp_status hip_status(hipError_t e) { return e == hipSuccess ? TP_MLP_OK : TP_MLP_ERR_HIP; }

const uint16_t* cu16(const void* p) { return static_cast<const uint16_t*>(p); }
uint16_t* u16(void* p) { return static_cast<uint16_t*>(p); }

// ----------------------------------------------------------------- launchers
uint32_t nbytes(int64_t rows, int64_t cols) { return (uint32_t)(rows * cols * 2); }

GemmArgs one_segment(int M, int N, int K) {
  GemmArgs g = {};
  g.M = M;
  g.N = N;
  g.nseg = 1;
  g.K[0] = K;
  return g;
}

hipError_t run_up_act(const Dims& d, const void* X, const void* W1, const void* Wg, void* A, void* U, void* G,
                      hipStream_t st) {
  GemmArgs g = one_segment((int)d.N, (int)d.Fi, (int)d.h);
  g.a[0] = g.a[1] = cu16(X);
  g.a_bytes[0] = g.a_bytes[1] = nbytes(d.N, d.h);
  g.lda = d.h;
  g.b_bytes[0] = g.b_bytes[1] = nbytes(d.h, d.Fi);
  g.ldb = d.Fi;
  g.c0 = A;
  g.ldc = d.Fi;
  if (d.act == ACT_SWIGLU) {
    g.b[0] = cu16(Wg);  // gate
    g.b[1] = cu16(W1);  // up
    g.e0 = G;
    g.e1 = U;
    return gemm_launch(GEMM_UP_SWIGLU, d.act, g, num_cu_current(), st);
  }
  g.b[0] = g.b[1] = cu16(W1);
  g.e0 = U;
  return gemm_launch(GEMM_UP_ACT, d.act, g, num_cu_current(), st);
}

hipError_t run_down(const Dims& d, const void* A, const void* W2, void* Y, hipStream_t st) {
  GemmArgs g = one_segment((int)d.N, (int)d.h, (int)d.Fi);
  g.a[0] = g.a[1] = cu16(A);
  g.a_bytes[0] = g.a_bytes[1] = nbytes(d.N, d.Fi);
  g.lda = d.Fi;
  g.b[0] = g.b[1] = cu16(W2);
  g.b_bytes[0] = g.b_bytes[1] = nbytes(d.Fi, d.h);
  g.ldb = d.h;
  g.c0 = Y;
  g.ldc = d.h;
  return gemm_launch(GEMM_DOWN, d.act, g, num_cu_current(), st);
}

GemmArgs dgrad_act_args(const Dims& d, const void* dY, const void* W2, const void* U, const void* G, void* dU) {
  GemmArgs g = one_segment((int)d.N, (int)d.Fi, (int)d.h);
  g.a[0] = g.a[1] = cu16(dY);
  g.a_bytes[0] = g.a_bytes[1] = nbytes(d.N, d.h);
  g.lda = d.h;
  g.b[0] = g.b[1] = cu16(W2);  // W2_i [F_i][h] is [n][k]
  g.b_bytes[0] = g.b_bytes[1] = nbytes(d.Fi, d.h);
  g.ldb = d.h;
  g.c0 = dU;
  g.lde = d.Fi;
  if (d.act == ACT_SWIGLU) {
    g.ldc = 2 * d.Fi;
    g.e0 = const_cast<void*>(G);
    g.e1 = const_cast<void*>(U);
  } else {
    g.ldc = d.Fi;
    g.e0 = const_cast<void*>(U);
  }
  return g;
}

hipError_t run_dgrad_act(const Dims& d, const void* dY, const void* W2, const void* U, const void* G, void* dU,
                         hipStream_t st) {
  return gemm_launch(GEMM_DGRAD_ACT, d.act, dgrad_act_args(d, dY, W2, U, G, dU), num_cu_current(), st);
}

GemmArgs wgrad_down_args(const Dims& d, const void* A, const void* dY, float* dW2) {
  GemmArgs g = one_segment((int)d.Fi, (int)d.h, (int)d.N);
  g.a[0] = g.a[1] = cu16(A);  // A_i [N][F_i] is [k][m]
  g.a_bytes[0] = g.a_bytes[1] = nbytes(d.N, d.Fi);
  g.lda = d.Fi;
  g.b[0] = g.b[1] = cu16(dY);  // dY [N][h] is [k][n]
  g.b_bytes[0] = g.b_bytes[1] = nbytes(d.N, d.h);
  g.ldb = d.h;
  g.c0 = g.c1 = dW2;
  g.ldc = d.h;
  g.c_split = (int)d.h;
  return g;
}

GemmArgs wgrad_up_args(const Dims& d, const void* X, const void* dU, float* dW1, float* dWg) {
  GemmArgs g = one_segment((int)d.h, (int)(d.g * d.Fi), (int)d.N);
  g.a[0] = g.a[1] = cu16(X);  // X [N][h] is [k][m]
  g.a_bytes[0] = g.a_bytes[1] = nbytes(d.N, d.h);
  g.lda = d.h;
  g.b[0] = g.b[1] = cu16(dU);  // dU [N][g*F_i] is [k][n]
  g.b_bytes[0] = g.b_bytes[1] = nbytes(d.N, d.g * d.Fi);
  g.ldb = d.g * d.Fi;
  g.c0 = d.act == ACT_SWIGLU ? dWg : dW1;  // columns [0, F_i): dG -> dWg
  g.c1 = dW1;                              // columns [F_i, 2F_i): dP -> dW_up
  g.ldc = d.Fi;
  g.c_split = (int)d.Fi;
  return g;
}

hipError_t run_wgrad_down(const Dims& d, const void* A, const void* dY, float* dW2, hipStream_t st) {
  return gemm_launch(GEMM_WGRAD, d.act, wgrad_down_args(d, A, dY, dW2), num_cu_current(), st);
}

hipError_t run_wgrad_up(const Dims& d, const void* X, const void* dU, float* dW1, float* dWg, hipStream_t st) {
  return gemm_launch(GEMM_WGRAD, d.act, wgrad_up_args(d, X, dU, dW1, dWg), num_cu_current(), st);
}

// The weight gradients of an empty batch are sums over no tokens: zero.
hipError_t zero_wgrads(const Dims& d, float* dW1, float* dWg, float* dW2, hipStream_t st) {
  const int64_t n = d.h * d.Fi;
  const int cu = num_cu_current();
  hipError_t e = zero_f32_launch(dW1, n, cu, st);
  if (e == hipSuccess) e = zero_f32_launch(dWg, n, cu, st);
  if (e == hipSuccess) e = zero_f32_launch(dW2, n, cu, st);
  return e;
}

// Both weight gradients in one launch: neither leaves a partial last wave of
// blocks on its own (each output element is summed over k in the same order
// as in the separate launches, so the results are bitwise the same).
hipError_t run_wgrads(const Dims& d, const void* X, const void* A, const void* dY, const void* dU, float* dW1,
                      float* dWg, float* dW2, hipStream_t st) {
  return gemm_launch2(GEMM_WGRAD, d.act, wgrad_down_args(d, A, dY, dW2), wgrad_up_args(d, X, dU, dW1, dWg),
                      num_cu_current(), st);
}

GemmArgs dgrad_up_args(const Dims& d, const void* dU, const void* W1, const void* Wg, void* dX) {
  GemmArgs g = one_segment((int)d.N, (int)d.h, (int)d.Fi);
  g.a[0] = g.a[1] = cu16(dU);
  g.a_bytes[0] = g.a_bytes[1] = nbytes(d.N, d.g * d.Fi);
  g.lda = d.g * d.Fi;
  g.b_bytes[0] = g.b_bytes[1] = nbytes(d.h, d.Fi);
  g.ldb = d.Fi;  // W [h][F_i] read as [n][k]
  if (d.act == ACT_SWIGLU) {
    // [dG | dP] @ [Wg_i | W1_i]^T as two k segments
    g.nseg = 2;
    g.K[1] = (int)d.Fi;
    g.a_koff[1] = (int)d.Fi;
    g.b[0] = cu16(Wg);
    g.b[1] = cu16(W1);
  } else {
    g.b[0] = g.b[1] = cu16(W1);
  }
  g.c0 = dX;
  g.ldc = d.h;
  return g;
}

hipError_t run_dgrad_up(const Dims& d, const void* dU, const void* W1, const void* Wg, void* dX, hipStream_t st) {
  return gemm_launch(GEMM_DGRAD, d.act, dgrad_up_args(d, dU, W1, Wg, dX), num_cu_current(), st);
}

// An input gradient and the weight gradient computed from the same inputs
// run as one mixed grid of 256x256 tiles when those tiles fill every CU at
// least once (gemm_launch_mixed); with fewer tiles, as two launches, each
// with its own tile choice.  Either way each element is summed over k in
// the same order, so the results are bitwise the same.
int64_t tiles256(const GemmArgs& g) { return (int64_t)((g.M + 255) / 256) * ((g.N + 255) / 256); }
hipError_t run_pair(GemmKind kp, int act, const GemmArgs& p, const GemmArgs& q, hipStream_t st) {
  const int ncu = num_cu_current();
  if (tiles256(p) + tiles256(q) >= ncu) return gemm_launch_mixed(kp, act, p, q, nullptr, st);
  hipError_t e = gemm_launch(kp, act, p, ncu, st);
  if (e == hipSuccess) e = gemm_launch(GEMM_WGRAD, act, q, ncu, st);
  return e;
}

// With few tokens (1 <= N <= SK_MAX_N) the input gradients have a handful of
// row tiles but a long k: they run as the small-batch split-K product, whose
// float32 partials live in the weight gradient's storage (the same call
// writes it only afterwards), with at most as many k-splits as fit there.
// The weight gradient (k = N) then runs on the wide tiles.
bool small_bwd(const Dims& d) { return d.N >= 1 && d.N <= SK_MAX_N; }

// dU on the split-K kernel, its partials [ks][N][F_i] in dW2 [F_i][h] (ks <= h / N)
hipError_t run_down_dgrad_small(const Dims& d, const void* dY, const void* W2, const void* U, const void* G, void* dU,
                                float* dW2, hipStream_t st) {
  const SkinnyPlan p = skinny_plan((int)d.N, (int)d.h, (int)d.Fi, 1, SKINNY_TARGET_BLOCKS, (int)(d.h / d.N));
  return skinny_dgrad_act_launch(d.act, (int)d.N, cu16(dY), cu16(W2), (int)d.h, (int)d.Fi, p, dW2, cu16(U), cu16(G),
                                 u16(dU), st);
}

// dX on the split-K kernel, its partials [ks][g][N][h] in dW1 [h][F_i] (ks <= F_i / (g N))
hipError_t run_up_dgrad_small(const Dims& d, const void* dU, const void* W1, const void* Wg, void* dX, float* dW1,
                              hipStream_t st) {
  const SkinnyPlan p =
      skinny_plan((int)d.N, (int)d.Fi, (int)d.h, d.g, SKINNY_TARGET_BLOCKS, (int)(d.Fi / (d.g * d.N)));
  return skinny_dgrad_up_launch(d.act, (int)d.N, cu16(dU), cu16(W1), cu16(Wg), (int)d.h, (int)d.Fi, p, dW1, u16(dX),
                                st);
}

// The down-projection's backward: dU (dgrad through W2 with the activation
// derivative) and dW2 = A_i^T dY.
hipError_t run_down_bwd(const Dims& d, const void* dY, const void* W2, const void* U, const void* G, const void* A,
                        void* dU, float* dW2, hipStream_t st) {
  if (small_bwd(d) && d.h >= d.N) {
    hipError_t e = run_down_dgrad_small(d, dY, W2, U, G, dU, dW2, st);
    if (e == hipSuccess) e = gemm_launch(GEMM_WGRAD, d.act, wgrad_down_args(d, A, dY, dW2), num_cu_current(), st);
    return e;
  }
  return run_pair(GEMM_DGRAD_ACT, d.act, dgrad_act_args(d, dY, W2, U, G, dU), wgrad_down_args(d, A, dY, dW2), st);
}

// The up-projection's backward: dX_partial = dU W1_i^T and dW1 (dWg) = X^T dU.
hipError_t run_up_bwd(const Dims& d, const void* X, const void* dU, const void* W1, const void* Wg, void* dX,
                      float* dW1, float* dWg, hipStream_t st) {
  if (small_bwd(d) && d.Fi >= d.g * d.N) {
    hipError_t e = run_up_dgrad_small(d, dU, W1, Wg, dX, dW1, st);
    if (e == hipSuccess) e = gemm_launch(GEMM_WGRAD, d.act, wgrad_up_args(d, X, dU, dW1, dWg), num_cu_current(), st);
    return e;
  }
  return run_pair(GEMM_DGRAD, d.act, dgrad_up_args(d, dU, W1, Wg, dX), wgrad_up_args(d, X, dU, dW1, dWg), st);
}

// ------------------------------------------------------- attention projections
struct AttnDims {
  int64_t N, h;
  int64_t q_cols, kv_cols, qkv_cols;  // this rank's query / key-value / fused widths
};

// INVALID_ARG for a malformed shape or head split, UNSUPPORTED for t above
// MAX_T or an operand too large for one buffer resource.
tp_mlp_status attn_status(const tp_attn_shape* s, AttnDims& a) {
  if (s == nullptr) return TP_MLP_ERR_INVALID_ARG;
  if (s->t < 1 || s->rank < 0 || s->rank >= s->t) return TP_MLP_ERR_INVALID_ARG;
  if (s->n_tokens < 0 || s->hidden < 8 || s->hidden % 8 != 0) return TP_MLP_ERR_INVALID_ARG;
  if (s->n_heads < 1 || s->n_kv_heads < 1 || s->head_dim < 8 || s->head_dim % 8 != 0) return TP_MLP_ERR_INVALID_ARG;
  const int64_t t = s->t, nh = s->n_heads, nkv = s->n_kv_heads, d = s->head_dim;
  if (nh % nkv != 0 || nh % t != 0) return TP_MLP_ERR_INVALID_ARG;
  if (nkv >= t ? nkv % t != 0 : t % nkv != 0) return TP_MLP_ERR_INVALID_ARG;
  if (t > MAX_T) return TP_MLP_ERR_UNSUPPORTED;
  a.N = s->n_tokens;
  a.h = s->hidden;
  a.q_cols = nh / t * d;
  a.kv_cols = (nkv >= t ? nkv / t : 1) * d;
  a.qkv_cols = a.q_cols + 2 * a.kv_cols;
  const int64_t lim = 0x7fffffffLL;
  if (a.N > lim || a.h > lim || a.qkv_cols > lim) return TP_MLP_ERR_UNSUPPORTED;
  const uint64_t cap = GEMM_MAX_OPERAND_BYTES / 2;
  const uint64_t N = (uint64_t)a.N, h = (uint64_t)a.h, w = (uint64_t)a.qkv_cols;
  if (N * h > cap || N * w > cap || h * w > cap) return TP_MLP_ERR_UNSUPPORTED;
  return TP_MLP_OK;
}

// 1 <= N <= SK_MAX_N tokens: the forward projections stream their weights
// once through the split-K small-batch product instead of wide tiles.
bool attn_small(const AttnDims& a) { return a.N >= 1 && a.N <= SK_MAX_N; }
SkinnyPlan attn_qkv_plan(const AttnDims& a) {
  return skinny_plan((int)a.N, (int)a.h, (int)a.qkv_cols, 1, SKINNY_TARGET_BLOCKS, INT_MAX);
}
SkinnyPlan attn_out_plan(const AttnDims& a) {
  return skinny_plan((int)a.N, (int)a.q_cols, (int)a.h, 1, SKINNY_TARGET_BLOCKS, INT_MAX);
}
size_t attn_workspace(const AttnDims& a) {
  if (!attn_small(a)) return 0;
  const size_t q = attn_qkv_plan(a).part_floats, o = attn_out_plan(a).part_floats;
  return round256((q > o ? q : o) * sizeof(float));
}
bool disjoint(const void* a, uint64_t na, const void* b, uint64_t nb);

// The small-batch path's workspace: present, large enough, aligned, and
// disjoint from the output.
tp_mlp_status attn_ws_status(const AttnDims& a, void* workspace, size_t workspace_bytes, const void* out,
                             uint64_t out_bytes) {
  const size_t need = attn_workspace(a);
  if (need == 0) return TP_MLP_OK;
  if (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)) return TP_MLP_ERR_WORKSPACE;
  if (!disjoint(workspace, need, out, out_bytes)) return TP_MLP_ERR_INVALID_ARG;
  return TP_MLP_OK;
}

// C [M, Nc] = A [M, K] @ B [K, Nc], both row-major, bf16 out.
hipError_t run_nn(int64_t M, int64_t Nc, int64_t K, const void* A, const void* B, void* C, hipStream_t st) {
  GemmArgs g = one_segment((int)M, (int)Nc, (int)K);
  g.a[0] = g.a[1] = cu16(A);
  g.a_bytes[0] = g.a_bytes[1] = nbytes(M, K);
  g.lda = K;
  g.b[0] = g.b[1] = cu16(B);
  g.b_bytes[0] = g.b_bytes[1] = nbytes(K, Nc);
  g.ldb = Nc;
  g.c0 = C;
  g.ldc = Nc;
  return gemm_launch(GEMM_DOWN, 0, g, num_cu_current(), st);
}

// k-slices for an NT product whose 256x192 tile grid fills at most half of
// the CUs: up to one block per CU, at least NT_SPLIT_MIN_K of k per slice
// (whole 64-deep k-tiles), at most NT_SPLIT_MAX slices.  0: no split.
constexpr int NT_SPLIT_MIN_K = 1024;
constexpr int NT_SPLIT_MAX = 8;
int nt_slices(int64_t M, int64_t Nc, int64_t K, int num_cu) {
  const int64_t tiles = ((M + 255) / 256) * ((Nc + 191) / 192);
  if (tiles * 2 > num_cu) return 0;
  int64_t s = num_cu / tiles;
  if (s > K / NT_SPLIT_MIN_K) s = K / NT_SPLIT_MIN_K;
  if (s > NT_SPLIT_MAX) s = NT_SPLIT_MAX;
  return s >= 2 ? (int)s : 0;
}

// An NT product with 1 <= M <= SK_MAX_N rows may run on the small-batch
// split-K kernel with at most skinny_cap k-splits (the number the weight
// gradient's storage holds, passed alike by every call that must give the
// same bits), and does while its partials, written and read back
// (2 ks M Nc 4 bytes), stay below the weight's bytes (K Nc 2): past that the
// wide tiles, themselves split along k when their grid is small, were as
// fast or faster on the attention projections' input gradients (70B widths
// at 128 tokens: dO 43 against 36 us).
bool skinny_nt_pays(const SkinnyPlan& p, int64_t M, int64_t K) { return 4 * (int64_t)p.ks * M < K; }
int cap_of(int64_t storage_floats, int64_t M, int64_t Nc) {
  return (int)std::min<int64_t>(storage_floats / (M * Nc), INT_MAX);
}

// C [M, Nc] = A [M, K] @ B^T with B stored [Nc, K], bf16 out.  With few rows
// and room in `part` (device, float32, part_floats of them, no contents
// needed), the small-batch split-K product as above; else, when the tile grid
// leaves most CUs idle and `part` holds slices * M * Nc partials, the product
// runs split along k into float32 partials, whose sum in slice order is
// rounded to bf16 once.
hipError_t run_nt(int64_t M, int64_t Nc, int64_t K, const void* A, const void* B, void* C, hipStream_t st,
                  float* part = nullptr, uint64_t part_floats = 0, int skinny_cap = 0) {
  if (part && skinny_cap >= 1 && M >= 1 && M <= SK_MAX_N) {
    const SkinnyPlan p = skinny_plan((int)M, (int)K, (int)Nc, 1, SKINNY_TARGET_BLOCKS, skinny_cap);
    if (skinny_nt_pays(p, M, K) && p.part_floats <= part_floats)
      return skinny_product_launch((int)M, cu16(A), cu16(B), (int)K, (int)Nc, p, part, u16(C), st, true);
  }
  const int ncu = num_cu_current();
  const int s = part ? nt_slices(M, Nc, K, ncu) : 0;
  if (s > 0 && (uint64_t)s * (uint64_t)M * (uint64_t)Nc <= part_floats) {
    GemmArgs g = one_segment((int)M, (int)Nc, (int)K);
    g.a[0] = g.a[1] = cu16(A);
    g.a_bytes[0] = g.a_bytes[1] = nbytes(M, K);
    g.lda = K;
    g.b[0] = g.b[1] = cu16(B);
    g.b_bytes[0] = g.b_bytes[1] = nbytes(Nc, K);
    g.ldb = K;
    g.kslice = (int)(((K + s - 1) / s + 63) / 64 * 64);
    const int slices = (int)((K + g.kslice - 1) / g.kslice);
    g.c0 = part;
    g.ldc = Nc;
    g.c_slice = M * Nc;
    hipError_t e = gemm_launch(GEMM_NT_SPLITK, 0, g, ncu, st);
    if (e != hipSuccess) return e;
    return ksum_launch(part, slices, M * Nc, u16(C), st);
  }
  GemmArgs g = one_segment((int)M, (int)Nc, (int)K);
  g.a[0] = g.a[1] = cu16(A);
  g.a_bytes[0] = g.a_bytes[1] = nbytes(M, K);
  g.lda = K;
  g.b[0] = g.b[1] = cu16(B);
  g.b_bytes[0] = g.b_bytes[1] = nbytes(Nc, K);
  g.ldb = K;
  g.c0 = C;
  g.ldc = Nc;
  return gemm_launch(GEMM_DGRAD, 0, g, num_cu_current(), st);
}

// C [M, Nc] = A^T @ B with A stored [K, M] and B stored [K, Nc], fp32 out.
hipError_t run_tn(int64_t M, int64_t Nc, int64_t K, const void* A, const void* B, float* C, hipStream_t st) {
  GemmArgs g = one_segment((int)M, (int)Nc, (int)K);
  g.a[0] = g.a[1] = cu16(A);
  g.a_bytes[0] = g.a_bytes[1] = nbytes(K, M);
  g.lda = M;
  g.b[0] = g.b[1] = cu16(B);
  g.b_bytes[0] = g.b_bytes[1] = nbytes(K, Nc);
  g.ldb = Nc;
  g.c0 = g.c1 = C;
  g.ldc = Nc;
  g.c_split = (int)Nc;
  return gemm_launch(GEMM_WGRAD, 0, g, num_cu_current(), st);
}

// The unsplit NT product of run_nt and the TN product of run_tn as GEMM
// arguments (for the mixed launches).
GemmArgs nt_args(int64_t M, int64_t Nc, int64_t K, const void* A, const void* B, void* C) {
  GemmArgs g = one_segment((int)M, (int)Nc, (int)K);
  g.a[0] = g.a[1] = cu16(A);
  g.a_bytes[0] = g.a_bytes[1] = nbytes(M, K);
  g.lda = K;
  g.b[0] = g.b[1] = cu16(B);
  g.b_bytes[0] = g.b_bytes[1] = nbytes(Nc, K);
  g.ldb = K;
  g.c0 = C;
  g.ldc = Nc;
  return g;
}
GemmArgs tn_args(int64_t M, int64_t Nc, int64_t K, const void* A, const void* B, float* C) {
  GemmArgs g = one_segment((int)M, (int)Nc, (int)K);
  g.a[0] = g.a[1] = cu16(A);
  g.a_bytes[0] = g.a_bytes[1] = nbytes(K, M);
  g.lda = M;
  g.b[0] = g.b[1] = cu16(B);
  g.b_bytes[0] = g.b_bytes[1] = nbytes(K, Nc);
  g.ldb = Nc;
  g.c0 = g.c1 = C;
  g.ldc = Nc;
  g.c_split = (int)Nc;
  return g;
}

// The attention QKV projection's backward: dX = dQKV Wqkv^T and dWqkv =
// X^T dQKV, and (dWo_i non-NULL) the output projection's weight gradient
// dWo = O^T dY, deferred to share the launch.  One mixed grid when the
// 256x256 tiles fill every CU at least once; otherwise dX (split along k
// into part_floats of part when its tiles leave most CUs idle) and then the
// weight gradients.
hipError_t run_attn_qkv_bwd(const AttnDims& a, const void* X, const void* Wqkv, const void* dQKV, float* dWqkv,
                            void* dX, const void* dY, const void* O, float* dWo, float* part, uint64_t part_floats,
                            hipStream_t st) {
  const GemmArgs p = nt_args(a.N, a.h, a.qkv_cols, dQKV, Wqkv, dX);
  const GemmArgs q0 = tn_args(a.h, a.qkv_cols, a.N, X, dQKV, dWqkv);
  GemmArgs q1 = q0;
  if (dWo) q1 = tn_args(a.q_cols, a.h, a.N, O, dY, dWo);
  const int cap = part && a.N >= 1 ? cap_of((int64_t)part_floats, a.N, a.h) : 0;
  if (cap >= 1 && a.N <= SK_MAX_N &&
      skinny_nt_pays(skinny_plan((int)a.N, (int)a.qkv_cols, (int)a.h, 1, SKINNY_TARGET_BLOCKS, cap), a.N,
                     a.qkv_cols)) {
    // few tokens: dX as the split-K product, then the weight gradient(s) in one launch
    hipError_t e = run_nt(a.N, a.h, a.qkv_cols, dQKV, Wqkv, dX, st, part, part_floats, cap);
    if (e != hipSuccess) return e;
    return dWo ? gemm_launch2(GEMM_WGRAD, 0, q0, q1, num_cu_current(), st)
               : gemm_launch(GEMM_WGRAD, 0, q0, num_cu_current(), st);
  }
  if (tiles256(p) + tiles256(q0) + (dWo ? tiles256(q1) : 0) >= num_cu_current())
    return gemm_launch_mixed(GEMM_DGRAD, 0, p, q0, dWo ? &q1 : nullptr, st);
  hipError_t e = run_nt(a.N, a.h, a.qkv_cols, dQKV, Wqkv, dX, st, part, part_floats);
  if (e == hipSuccess) e = gemm_launch(GEMM_WGRAD, 0, q0, num_cu_current(), st);
  if (e == hipSuccess && dWo) e = gemm_launch(GEMM_WGRAD, 0, q1, num_cu_current(), st);
  return e;
}

// k-splits of dO = dY Wo^T on the small-batch kernel: as many as dW_o's
// storage holds (h / N), in tp_attn_out_bwd_shard and tp_attn_out_dgrad_shard
// alike.
int dO_cap(const AttnDims& a) { return a.N >= 1 ? cap_of(a.q_cols * a.h, a.N, a.q_cols) : 0; }

// Float32 partials the output projection's input gradient dO = dY Wo^T
// splits into along k (0: not split).  With few tokens, the small-batch
// plan with as many splits as dW_o's storage would hold (h / N), the plan
// tp_attn_out_bwd_shard runs, so that both give the same dO.
uint64_t attn_dO_part_floats(const AttnDims& a) {
  if (a.N >= 1 && a.N <= SK_MAX_N && a.h >= a.N) {
    const SkinnyPlan p = skinny_plan((int)a.N, (int)a.h, (int)a.q_cols, 1, SKINNY_TARGET_BLOCKS, dO_cap(a));
    if (skinny_nt_pays(p, a.N, a.h)) return p.part_floats;
  }
  const int s = nt_slices(a.N, a.q_cols, a.h, num_cu_current());
  return s > 0 ? (uint64_t)s * (uint64_t)a.N * (uint64_t)a.q_cols : 0;
}

// Extents of a [rows, cols] block for the streaming kernels (reductions,
// gather, column sums): cols / 8 is an int there, and byte counts of the
// block must not overflow 64 bits.  rows may be 0 (an empty block).
// INVALID_ARG for a malformed shape, UNSUPPORTED above these limits.
constexpr int64_t STREAM_MAX_COLS = (int64_t)1 << 33;
constexpr int64_t STREAM_MAX_ELEMS = (int64_t)1 << 50;
tp_mlp_status block_status(int64_t rows, int64_t cols) {
  if (rows < 0 || cols < 8 || cols % 8 != 0) return TP_MLP_ERR_INVALID_ARG;
  if (cols > STREAM_MAX_COLS || rows > STREAM_MAX_ELEMS / cols) return TP_MLP_ERR_UNSUPPORTED;
  return TP_MLP_OK;
}

// A host array of t device pointers to bf16 [rows, cols] blocks: INVALID_ARG
// for a malformed list or shape, UNSUPPORTED for t above MAX_T or a block
// beyond the streaming limits.
tp_mlp_status partial_list(int32_t t, const void* const* ptrs, int64_t rows, int64_t cols, PartialPtrs& pp) {
  if (ptrs == nullptr || t < 1) return TP_MLP_ERR_INVALID_ARG;
  if (t > MAX_T) return TP_MLP_ERR_UNSUPPORTED;
  if (const tp_mlp_status bs = block_status(rows, cols)) return bs;
  const uint64_t bytes = (uint64_t)rows * (uint64_t)cols * 2;
  for (int r = 0; r < t; ++r) {
    if (!req_n(ptrs[r], bytes)) return TP_MLP_ERR_INVALID_ARG;
    pp.p[r] = cu16(ptrs[r]);
  }
  return TP_MLP_OK;
}

// Byte ranges [a, a+na) and [b, b+nb) do not overlap (an empty range never does).
bool disjoint(const void* a, uint64_t na, const void* b, uint64_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return na == 0 || nb == 0 || x + na <= y || y + nb <= x;
}
// ...or coincide exactly.
bool same_or_disjoint(const void* a, uint64_t na, const void* b, uint64_t nb) {
  return (a == b && na == nb) || disjoint(a, na, b, nb);
}

// A device buffer of n bytes (p may be NULL: an absent optional buffer).
struct Span {
  const void* p;
  uint64_t n;
};
// The outputs are pairwise disjoint and disjoint from every input.
bool spans_ok(std::initializer_list<Span> outs, std::initializer_list<Span> ins) {
  for (auto o = outs.begin(); o != outs.end(); ++o) {
    if (!o->p) continue;
    for (auto q = o + 1; q != outs.end(); ++q)
      if (q->p && !disjoint(o->p, o->n, q->p, q->n)) return false;
    for (const Span& i : ins)
      if (i.p && !disjoint(o->p, o->n, i.p, i.n)) return false;
  }
  return true;
}

// The reduce-scatter's arguments: rank's block of rows/t rows, out may
// coincide exactly with the residual or with rank's block of any partial and
// must not otherwise overlap an input.
tp_mlp_status rs_status(int32_t t, const void* const* partials, int64_t rows, int64_t cols, int32_t rank,
                        const void* bias, const void* residual, const void* out, PartialPtrs& pp) {
  if (const tp_mlp_status ss = partial_list(t, partials, rows, cols, pp)) return ss;
  if (rows % t != 0 || rank < 0 || rank >= t) return TP_MLP_ERR_INVALID_ARG;
  const uint64_t out_bytes = (uint64_t)(rows / t) * (uint64_t)cols * 2;
  if (!req_n(out, out_bytes) || !opt_aligned(bias) || !opt_aligned(residual)) return TP_MLP_ERR_INVALID_ARG;
  const uint64_t block_off = (uint64_t)rank * out_bytes;
  for (int r = 0; r < t; ++r) {
    const uint8_t* blk = reinterpret_cast<const uint8_t*>(pp.p[r]) + block_off;
    if (!same_or_disjoint(out, out_bytes, blk, out_bytes)) return TP_MLP_ERR_INVALID_ARG;
    if (!disjoint(out, out_bytes, pp.p[r], block_off) ||
        !disjoint(out, out_bytes, blk + out_bytes, (uint64_t)(t - 1 - rank) * out_bytes))
      return TP_MLP_ERR_INVALID_ARG;
  }
  if (residual && !same_or_disjoint(out, out_bytes, residual, out_bytes)) return TP_MLP_ERR_INVALID_ARG;
  if (bias && !disjoint(out, out_bytes, bias, (uint64_t)cols * 2)) return TP_MLP_ERR_INVALID_ARG;
  return TP_MLP_OK;
}

// LayerNorm sizes and parameters shared by the sequence-parallel entry points.
tp_mlp_status ln_status(int64_t rows, int64_t cols, float eps, const void* gamma, const void* beta) {
  if (rows < 0 || rows >= (int64_t)1 << 31 || cols < 8 || cols % 8 != 0) return TP_MLP_ERR_INVALID_ARG;
  if (!(eps > 0.0f) || !(eps < 3.0e38f)) return TP_MLP_ERR_INVALID_ARG;
  if (!req(gamma) || !opt_aligned(beta)) return TP_MLP_ERR_INVALID_ARG;
  if (cols > LN_MAX_COLS) return TP_MLP_ERR_UNSUPPORTED;
  return TP_MLP_OK;
}

// The LayerNorm stash: both float32 [rows] or both NULL; disjoint from y and
// from each other.
bool stash_ok(const float* mean, const float* rstd, int64_t rows, const void* y, uint64_t y_bytes) {
  if (rows == 0) return opt_aligned(mean) && opt_aligned(rstd);
  if ((mean == nullptr) != (rstd == nullptr)) return false;
  if (!mean) return true;
  const uint64_t sb = (uint64_t)rows * 4;
  return req_n(mean, sb) && req_n(rstd, sb) && disjoint(mean, sb, rstd, sb) && disjoint(mean, sb, y, y_bytes) &&
         disjoint(rstd, sb, y, y_bytes);
}

}  // namespace

extern "C" {

const char* tp_mlp_status_string(tp_mlp_status st) {
  // a C caller may pass any int: read it as one (an out-of-range value of
  // the enum type would be undefined in C++)
  int v;
  std::memcpy(&v, &st, sizeof v);
  switch (v) {
    case TP_MLP_OK: return "ok";
    case TP_MLP_ERR_INVALID_ARG: return "invalid argument (pointer, shape, alignment, rank or activation)";
    case TP_MLP_ERR_UNSUPPORTED: return "valid but unsupported option";
    case TP_MLP_ERR_WORKSPACE: return "workspace missing or too small";
    case TP_MLP_ERR_HIP: return "HIP launch or query failed";
  }
  return "unknown status";
}

size_t tp_mlp_workspace_bytes(const tp_mlp_shape* s, int backward) {
  Dims d;
  if (!check_shape(s, d) || d.N == 0) return 0;
  if (backward) return col_sum_workspace_bytes(d.N, d.h);
  if (d.N == 1) return decode_layout(d).total;
  if (small_batch(d)) return skinny_layout(d).total;
  return 0;
}

size_t tp_mlp_bias_grad_workspace_bytes(int64_t rows, int64_t cols) {
  if (block_status(rows, cols) != TP_MLP_OK || rows == 0) return 0;
  return col_sum_workspace_bytes(rows, cols);
}

tp_mlp_status tp_mlp_up_act_shard(const tp_mlp_shape* s, const void* X, const void* W1_i, const void* Wg_i,
                                  void* A_i, void* U_i, void* G_i, hipStream_t stream) {
  Dims d;
  if (const tp_mlp_status ss = shape_status(s, d)) return ss;
  const bool sw = d.act == ACT_SWIGLU;
  const uint64_t x = (uint64_t)d.N * d.h * 2, w = (uint64_t)d.h * d.Fi * 2, a = (uint64_t)d.N * d.Fi * 2;
  if (!req_n(X, x) || !req(W1_i) || !req_n(A_i, a) || !opt_aligned(U_i) || !opt_aligned(G_i))
    return TP_MLP_ERR_INVALID_ARG;
  if (sw != (Wg_i != nullptr) || !opt_aligned(Wg_i)) return TP_MLP_ERR_INVALID_ARG;
  if (!sw && G_i != nullptr) return TP_MLP_ERR_INVALID_ARG;
  if (sw && d.N > 0 && ((U_i == nullptr) != (G_i == nullptr))) return TP_MLP_ERR_INVALID_ARG;
  if (!spans_ok({{A_i, a}, {U_i, a}, {G_i, a}}, {{X, x}, {W1_i, w}, {Wg_i, w}})) return TP_MLP_ERR_INVALID_ARG;
  if (d.N == 0) return TP_MLP_OK;
  return hip_status(run_up_act(d, X, W1_i, Wg_i, A_i, U_i, G_i, stream));
}

tp_mlp_status tp_mlp_down_shard(const tp_mlp_shape* s, const void* A_i, const void* W2_i, void* Y_i,
                                hipStream_t stream) {
  Dims d;
  if (const tp_mlp_status ss = shape_status(s, d)) return ss;
  const uint64_t y = (uint64_t)d.N * d.h * 2, a = (uint64_t)d.N * d.Fi * 2;
  if (!req_n(A_i, a) || !req(W2_i) || !req_n(Y_i, y)) return TP_MLP_ERR_INVALID_ARG;
  if (!spans_ok({{Y_i, y}}, {{A_i, a}, {W2_i, (uint64_t)d.Fi * d.h * 2}})) return TP_MLP_ERR_INVALID_ARG;
  if (d.N == 0) return TP_MLP_OK;
  return hip_status(run_down(d, A_i, W2_i, Y_i, stream));
}

}  // extern "C"

namespace {

// The forward's argument checks; the scratch the shape needs (0 for the
// wide-tile path) in need_bytes.
tp_mlp_status fwd_check(const tp_mlp_shape* s, const void* X, const void* W1_i, const void* Wg_i, const void* W2_i,
                        const void* Y_i, const void* A_i, const void* U_i, const void* G_i, const void* workspace,
                        Dims& d, size_t& need_bytes) {
  if (const tp_mlp_status ss = shape_status(s, d)) return ss;
  const bool sw = d.act == ACT_SWIGLU;
  const uint64_t x = (uint64_t)d.N * d.h * 2, w = (uint64_t)d.h * d.Fi * 2, a = (uint64_t)d.N * d.Fi * 2;
  if (!req_n(X, x) || !req(W1_i) || !req(W2_i) || !req_n(Y_i, x) || !req_n(A_i, a)) return TP_MLP_ERR_INVALID_ARG;
  if (!opt_aligned(U_i) || !opt_aligned(G_i) || !opt_aligned(Wg_i) || !opt_aligned(workspace))
    return TP_MLP_ERR_INVALID_ARG;
  if (sw != (Wg_i != nullptr)) return TP_MLP_ERR_INVALID_ARG;
  if (!sw && G_i != nullptr) return TP_MLP_ERR_INVALID_ARG;
  if (sw && d.N > 0 && ((U_i == nullptr) != (G_i == nullptr))) return TP_MLP_ERR_INVALID_ARG;
  need_bytes = d.N == 1 ? decode_layout(d).total : (small_batch(d) ? skinny_layout(d).total : 0);
  if (!spans_ok({{Y_i, x}, {A_i, a}, {U_i, a}, {G_i, a}, {need_bytes ? workspace : nullptr, need_bytes}},
                {{X, x}, {W1_i, w}, {Wg_i, w}, {W2_i, w}}))
    return TP_MLP_ERR_INVALID_ARG;
  return TP_MLP_OK;
}

// The forward's launches, after fwd_check: the workspace (when the shape
// needs one) is device memory of at least the needed size.
tp_mlp_status fwd_run(const Dims& d, const void* X, const void* W1_i, const void* Wg_i, const void* W2_i, void* Y_i,
                      void* A_i, void* U_i, void* G_i, void* workspace, hipStream_t stream) {
  const bool sw = d.act == ACT_SWIGLU;
  if (d.N == 0) return TP_MLP_OK;  // no tokens: nothing to compute
  if (d.N == 1) {
    const DecodeLayout L = decode_layout(d);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    float* part_up = reinterpret_cast<float*>(ws + L.off_part_up);
    float* part_dn = reinterpret_cast<float*>(ws + L.off_part_down);
    int* cnt = reinterpret_cast<int*>(ws + L.off_cnt);
    return hip_status(decode_launch(d.act, cu16(X), cu16(sw ? Wg_i : W1_i), cu16(W1_i), cu16(W2_i), (int)d.h,
                                    (int)d.Fi, L.up, L.down, part_up, part_dn, cnt, u16(A_i), u16(sw ? G_i : U_i),
                                    u16(sw ? U_i : nullptr), u16(Y_i), stream));
  }
  if (small_batch(d)) {
    const SkinnyLayout L = skinny_layout(d);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    return hip_status(skinny_launch(d.act, (int)d.N, cu16(X), cu16(sw ? Wg_i : W1_i), cu16(W1_i), cu16(W2_i),
                                    (int)d.h, (int)d.Fi, L.up, L.down, reinterpret_cast<float*>(ws + L.off_part_up),
                                    reinterpret_cast<float*>(ws + L.off_part_down), u16(A_i), u16(sw ? G_i : U_i),
                                    u16(sw ? U_i : nullptr), u16(Y_i), stream));
  }
  hipError_t e = run_up_act(d, X, W1_i, Wg_i, A_i, U_i, G_i, stream);
  if (e != hipSuccess) return TP_MLP_ERR_HIP;
  return hip_status(run_down(d, A_i, W2_i, Y_i, stream));
}

}  // namespace

extern "C" {

tp_mlp_status tp_mlp_fwd_shard(const tp_mlp_shape* s, const void* X, const void* W1_i, const void* Wg_i,
                               const void* W2_i, void* Y_i, void* A_i, void* U_i, void* G_i, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
  Dims d;
  size_t need = 0;
  if (const tp_mlp_status st = fwd_check(s, X, W1_i, Wg_i, W2_i, Y_i, A_i, U_i, G_i, workspace, d, need)) return st;
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return TP_MLP_ERR_WORKSPACE;
  return fwd_run(d, X, W1_i, Wg_i, W2_i, Y_i, A_i, U_i, G_i, workspace, stream);
}

tp_mlp_status tp_mlp_fwd_shard_noalloc(const tp_mlp_shape* s, const void* X, const void* W1_i, const void* Wg_i,
                                       const void* W2_i, void* Y_i, void* A_i, void* U_i, void* G_i,
                                       hipStream_t stream) {
  Dims d;
  size_t need = 0;
  if (const tp_mlp_status st = fwd_check(s, X, W1_i, Wg_i, W2_i, Y_i, A_i, U_i, G_i, nullptr, d, need)) return st;
  if (need > STATIC_SCRATCH_BYTES) return TP_MLP_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0 && d.N > 0 && (ws = static_scratch_current()) == nullptr) return TP_MLP_ERR_HIP;
  return fwd_run(d, X, W1_i, Wg_i, W2_i, Y_i, A_i, U_i, G_i, ws, stream);
}

tp_mlp_status tp_mlp_down_dgrad_act_shard(const tp_mlp_shape* s, const void* dY, const void* W2_i, const void* U_i,
                                          const void* G_i, void* dU_i, hipStream_t stream) {
  Dims d;
  if (const tp_mlp_status ss = shape_status(s, d)) return ss;
  const bool sw = d.act == ACT_SWIGLU;
  const uint64_t a = (uint64_t)d.N * d.Fi * 2, y = (uint64_t)d.N * d.h * 2;
  if (!req_n(dY, y) || !req(W2_i) || !req_n(U_i, a) || !req_n(dU_i, a)) return TP_MLP_ERR_INVALID_ARG;
  if (sw ? !req_n(G_i, a) : G_i != nullptr) return TP_MLP_ERR_INVALID_ARG;
  if (!spans_ok({{dU_i, a * d.g}}, {{dY, y}, {W2_i, (uint64_t)d.Fi * d.h * 2}, {U_i, a}, {G_i, a}}))
    return TP_MLP_ERR_INVALID_ARG;
  if (d.N == 0) return TP_MLP_OK;
  return hip_status(run_dgrad_act(d, dY, W2_i, U_i, G_i, dU_i, stream));
}

tp_mlp_status tp_mlp_down_wgrad_shard(const tp_mlp_shape* s, const void* A_i, const void* dY, float* dW2_i,
                                      hipStream_t stream) {
  Dims d;
  if (const tp_mlp_status ss = shape_status(s, d)) return ss;
  const uint64_t a = (uint64_t)d.N * d.Fi * 2, y = (uint64_t)d.N * d.h * 2;
  if (!req_n(A_i, a) || !req_n(dY, y) || !req(dW2_i)) return TP_MLP_ERR_INVALID_ARG;
  if (!spans_ok({{dW2_i, (uint64_t)d.Fi * d.h * 4}}, {{A_i, a}, {dY, y}})) return TP_MLP_ERR_INVALID_ARG;
  if (d.N == 0) return hip_status(zero_f32_launch(dW2_i, d.Fi * d.h, num_cu_current(), stream));
  return hip_status(run_wgrad_down(d, A_i, dY, dW2_i, stream));
}

tp_mlp_status tp_mlp_up_wgrad_shard(const tp_mlp_shape* s, const void* X, const void* dU_i, float* dW1_i,
                                    float* dWg_i, hipStream_t stream) {
  Dims d;
  if (const tp_mlp_status ss = shape_status(s, d)) return ss;
  const bool sw = d.act == ACT_SWIGLU;
  const uint64_t x = (uint64_t)d.N * d.h * 2, du = (uint64_t)d.N * d.g * d.Fi * 2;
  if (!req_n(X, x) || !req_n(dU_i, du) || !req(dW1_i)) return TP_MLP_ERR_INVALID_ARG;
  if (sw ? !req(dWg_i) : dWg_i != nullptr) return TP_MLP_ERR_INVALID_ARG;
  const uint64_t w4 = (uint64_t)d.h * d.Fi * 4;
  if (!spans_ok({{dW1_i, w4}, {dWg_i, w4}}, {{X, x}, {dU_i, du}})) return TP_MLP_ERR_INVALID_ARG;
  if (d.N == 0) return hip_status(zero_wgrads(d, dW1_i, dWg_i, nullptr, stream));
  return hip_status(run_wgrad_up(d, X, dU_i, dW1_i, dWg_i, stream));
}

tp_mlp_status tp_mlp_wgrad_shard(const tp_mlp_shape* s, const void* X, const void* A_i, const void* dY,
                                 const void* dU_i, float* dW1_i, float* dWg_i, float* dW2_i, hipStream_t stream) {
  Dims d;
  if (const tp_mlp_status ss = shape_status(s, d)) return ss;
  const bool sw = d.act == ACT_SWIGLU;
  const uint64_t x = (uint64_t)d.N * d.h * 2, w4 = (uint64_t)d.h * d.Fi * 4;
  const uint64_t a = (uint64_t)d.N * d.Fi * 2, du = (uint64_t)d.N * d.g * d.Fi * 2;
  if (!req_n(X, x) || !req_n(A_i, a) || !req_n(dY, x) || !req_n(dU_i, du) || !req(dW1_i) || !req(dW2_i))
    return TP_MLP_ERR_INVALID_ARG;
  if (sw ? !req(dWg_i) : dWg_i != nullptr) return TP_MLP_ERR_INVALID_ARG;
  if (!spans_ok({{dW1_i, w4}, {dWg_i, w4}, {dW2_i, w4}}, {{X, x}, {A_i, a}, {dY, x}, {dU_i, du}}))
    return TP_MLP_ERR_INVALID_ARG;
  if (d.N == 0) return hip_status(zero_wgrads(d, dW1_i, dWg_i, dW2_i, stream));
  return hip_status(run_wgrads(d, X, A_i, dY, dU_i, dW1_i, dWg_i, dW2_i, stream));
}

tp_mlp_status tp_mlp_up_dgrad_shard(const tp_mlp_shape* s, const void* dU_i, const void* W1_i, const void* Wg_i,
                                    void* dX_partial, hipStream_t stream) {
  Dims d;
  if (const tp_mlp_status ss = shape_status(s, d)) return ss;
  const bool sw = d.act == ACT_SWIGLU;
  const uint64_t w = (uint64_t)d.h * d.Fi * 2, dx = (uint64_t)d.N * d.h * 2, du = (uint64_t)d.N * d.g * d.Fi * 2;
  if (!req_n(dU_i, du) || !req(W1_i) || !req_n(dX_partial, dx)) return TP_MLP_ERR_INVALID_ARG;
  if (sw ? !req(Wg_i) : Wg_i != nullptr) return TP_MLP_ERR_INVALID_ARG;
  if (!spans_ok({{dX_partial, dx}}, {{dU_i, du}, {W1_i, w}, {Wg_i, w}})) return TP_MLP_ERR_INVALID_ARG;
  if (d.N == 0) return TP_MLP_OK;
  return hip_status(run_dgrad_up(d, dU_i, W1_i, Wg_i, dX_partial, stream));
}

tp_mlp_status tp_mlp_down_bwd_shard(const tp_mlp_shape* s, const void* dY, const void* W2_i, const void* U_i,
                                    const void* G_i, const void* A_i, void* dU_i, float* dW2_i, hipStream_t stream) {
  Dims d;
  if (const tp_mlp_status ss = shape_status(s, d)) return ss;
  const bool sw = d.act == ACT_SWIGLU;
  const uint64_t a = (uint64_t)d.N * d.Fi * 2, y = (uint64_t)d.N * d.h * 2;
  if (!req_n(dY, y) || !req(W2_i) || !req_n(U_i, a) || !req_n(A_i, a) || !req_n(dU_i, a) || !req(dW2_i))
    return TP_MLP_ERR_INVALID_ARG;
  if (sw ? !req_n(G_i, a) : G_i != nullptr) return TP_MLP_ERR_INVALID_ARG;
  if (!spans_ok({{dU_i, a * d.g}, {dW2_i, (uint64_t)d.Fi * d.h * 4}},
                {{dY, y}, {W2_i, (uint64_t)d.Fi * d.h * 2}, {U_i, a}, {G_i, a}, {A_i, a}}))
    return TP_MLP_ERR_INVALID_ARG;
  if (d.N == 0) return hip_status(zero_f32_launch(dW2_i, d.Fi * d.h, num_cu_current(), stream));
  return hip_status(run_down_bwd(d, dY, W2_i, U_i, G_i, A_i, dU_i, dW2_i, stream));
}

tp_mlp_status tp_mlp_up_bwd_shard(const tp_mlp_shape* s, const void* X, const void* dU_i, const void* W1_i,
                                  const void* Wg_i, void* dX_partial, float* dW1_i, float* dWg_i,
                                  hipStream_t stream) {
  Dims d;
  if (const tp_mlp_status ss = shape_status(s, d)) return ss;
  const bool sw = d.act == ACT_SWIGLU;
  const uint64_t x = (uint64_t)d.N * d.h * 2, w = (uint64_t)d.h * d.Fi * 2, du = (uint64_t)d.N * d.g * d.Fi * 2;
  if (!req_n(X, x) || !req_n(dU_i, du) || !req(W1_i) || !req_n(dX_partial, x) || !req(dW1_i))
    return TP_MLP_ERR_INVALID_ARG;
  if (sw ? (!req(Wg_i) || !req(dWg_i)) : (Wg_i != nullptr || dWg_i != nullptr)) return TP_MLP_ERR_INVALID_ARG;
  if (!spans_ok({{dX_partial, x}, {dW1_i, w * 2}, {dWg_i, w * 2}}, {{X, x}, {dU_i, du}, {W1_i, w}, {Wg_i, w}}))
    return TP_MLP_ERR_INVALID_ARG;
  if (d.N == 0) return hip_status(zero_wgrads(d, dW1_i, dWg_i, nullptr, stream));
  return hip_status(run_up_bwd(d, X, dU_i, W1_i, Wg_i, dX_partial, dW1_i, dWg_i, stream));
}

tp_mlp_status tp_mlp_bias_grad(const void* dY, int64_t rows, int64_t cols, float* db2, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
  if (const tp_mlp_status bs = block_status(rows, cols)) return bs;
  const uint64_t y = (uint64_t)rows * cols * 2;
  if (!req_n(dY, y) || !req(db2) || !opt_aligned(workspace)) return TP_MLP_ERR_INVALID_ARG;
  if (rows == 0) {  // a sum over no rows
    if (!spans_ok({{db2, (uint64_t)cols * 4}}, {})) return TP_MLP_ERR_INVALID_ARG;
    return hip_status(zero_f32_launch(db2, cols, num_cu_current(), stream));
  }
  if (workspace == nullptr || workspace_bytes < col_sum_workspace_bytes(rows, cols)) return TP_MLP_ERR_WORKSPACE;
  if (!spans_ok({{db2, (uint64_t)cols * 4}, {workspace, col_sum_workspace_bytes(rows, cols)}}, {{dY, y}}))
    return TP_MLP_ERR_INVALID_ARG;
  return hip_status(col_sum_launch(cu16(dY), rows, cols, db2, static_cast<float*>(workspace), stream));
}

tp_mlp_status tp_mlp_bwd_shard(const tp_mlp_shape* s, const void* X, const void* W1_i, const void* Wg_i,
                               const void* W2_i, const void* dY, const void* A_i, const void* U_i, const void* G_i,
                               void* dU_i, float* dW1_i, float* dWg_i, float* dW2_i, void* dX_partial, float* db2,
                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  Dims d;
  if (const tp_mlp_status ss = shape_status(s, d)) return ss;
  const bool sw = d.act == ACT_SWIGLU;
  const uint64_t x = (uint64_t)d.N * d.h * 2, w = (uint64_t)d.h * d.Fi * 2, a = (uint64_t)d.N * d.Fi * 2;
  if (!req_n(X, x) || !req(W1_i) || !req(W2_i) || !req_n(dY, x) || !req_n(A_i, a) || !req_n(U_i, a) ||
      !req_n(dU_i, a) || !req(dW1_i) || !req(dW2_i) || !req_n(dX_partial, x) || !opt_aligned(db2) ||
      !opt_aligned(workspace))
    return TP_MLP_ERR_INVALID_ARG;
  if (sw ? (!req(Wg_i) || !req_n(G_i, a) || !req(dWg_i)) : (Wg_i != nullptr || G_i != nullptr || dWg_i != nullptr))
    return TP_MLP_ERR_INVALID_ARG;
  // the bias gradient needs scratch unless there are no tokens to sum
  const uint64_t ws_used = db2 && d.N > 0 ? col_sum_workspace_bytes(d.N, d.h) : 0;
  if (ws_used && (workspace == nullptr || workspace_bytes < ws_used)) return TP_MLP_ERR_WORKSPACE;
  if (!spans_ok({{dU_i, a * d.g}, {dW1_i, w * 2}, {dWg_i, w * 2}, {dW2_i, w * 2}, {dX_partial, x},
                 {db2, (uint64_t)d.h * 4}, {ws_used ? workspace : nullptr, ws_used}},
                {{X, x}, {W1_i, w}, {Wg_i, w}, {W2_i, w}, {dY, x}, {A_i, a}, {U_i, a}, {G_i, a}}))
    return TP_MLP_ERR_INVALID_ARG;

  if (d.N == 0) {  // no tokens: every gradient is a sum over an empty set
    hipError_t e = zero_wgrads(d, dW1_i, dWg_i, dW2_i, stream);
    if (e == hipSuccess) e = zero_f32_launch(db2, d.h, num_cu_current(), stream);
    return hip_status(e);
  }
  hipError_t e;
  const GemmArgs wd = wgrad_down_args(d, A_i, dY, dW2_i), wu = wgrad_up_args(d, X, dU_i, dW1_i, dWg_i);
  if (small_bwd(d) && d.h >= d.N && d.Fi >= d.g * d.N && tiles256(wd) + tiles256(wu) <= num_cu_current()) {
    // few tokens and small weights: both input gradients on the split-K kernel
    // (partials in dW2_i, then dW1_i, as in the step calls), then both weight
    // gradients in one launch, which alone would each leave most CUs idle
    e = run_down_dgrad_small(d, dY, W2_i, U_i, G_i, dU_i, dW2_i, stream);
    if (e == hipSuccess) e = run_up_dgrad_small(d, dU_i, W1_i, Wg_i, dX_partial, dW1_i, stream);
    if (e == hipSuccess) e = gemm_launch2(GEMM_WGRAD, d.act, wd, wu, num_cu_current(), stream);
  } else {
    e = run_down_bwd(d, dY, W2_i, U_i, G_i, A_i, dU_i, dW2_i, stream);
    if (e == hipSuccess) e = run_up_bwd(d, X, dU_i, W1_i, Wg_i, dX_partial, dW1_i, dWg_i, stream);
  }
  if (e == hipSuccess && db2 != nullptr)
    e = col_sum_launch(cu16(dY), d.N, d.h, db2, static_cast<float*>(workspace), stream);
  return hip_status(e);
}

tp_mlp_status tp_mlp_reduce_partials_local(int32_t t, const void* const* partials, int64_t rows, int64_t cols,
                                           const void* bias, void* out, hipStream_t stream) {
  PartialPtrs pp = {};
  if (const tp_mlp_status ss = partial_list(t, partials, rows, cols, pp)) return ss;
  const uint64_t bytes = (uint64_t)rows * (uint64_t)cols * 2;
  if (!req_n(out, bytes) || !opt_aligned(bias)) return TP_MLP_ERR_INVALID_ARG;
  for (int r = 0; r < t; ++r)
    if (!same_or_disjoint(out, bytes, pp.p[r], bytes)) return TP_MLP_ERR_INVALID_ARG;
  if (rows == 0) return TP_MLP_OK;
  return hip_status(
      reduce_partials_launch(pp, t, rows, cols, 0, cu16(bias), nullptr, u16(out), num_cu_current(), stream));
}

tp_mlp_status tp_mlp_reduce_scatter_local(int32_t t, const void* const* partials, int64_t rows, int64_t cols,
                                          int32_t rank, const void* bias, const void* residual, void* out,
                                          hipStream_t stream) {
  PartialPtrs pp = {};
  if (const tp_mlp_status ss = rs_status(t, partials, rows, cols, rank, bias, residual, out, pp)) return ss;
  const int64_t shard = rows / t;
  if (shard == 0) return TP_MLP_OK;
  return hip_status(reduce_partials_launch(pp, t, shard, cols, (int64_t)rank * shard, cu16(bias), cu16(residual),
                                           u16(out), num_cu_current(), stream));
}

tp_mlp_status tp_mlp_all_gather_local(int32_t t, const void* const* shards, int64_t shard_rows, int64_t cols,
                                      void* out, hipStream_t stream) {
  PartialPtrs pp = {};
  if (const tp_mlp_status ss = partial_list(t, shards, shard_rows, cols, pp)) return ss;
  const uint64_t shard_bytes = (uint64_t)shard_rows * (uint64_t)cols * 2;
  if (!req_n(out, shard_bytes)) return TP_MLP_ERR_INVALID_ARG;
  for (int r = 0; r < t; ++r)
    if (!disjoint(out, shard_bytes * (uint64_t)t, pp.p[r], shard_bytes)) return TP_MLP_ERR_INVALID_ARG;
  if (shard_rows == 0) return TP_MLP_OK;
  return hip_status(gather_launch(pp, t, shard_rows, cols, u16(out), num_cu_current(), stream));
}

size_t tp_attn_workspace_bytes(const tp_attn_shape* s) {
  AttnDims a;
  if (attn_status(s, a) != TP_MLP_OK) return 0;
  return attn_workspace(a);
}

tp_mlp_status tp_attn_qkv_shard(const tp_attn_shape* s, const void* X, const void* Wqkv_i, void* QKV_i,
                                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  AttnDims a;
  if (const tp_mlp_status ss = attn_status(s, a)) return ss;
  if (!req_n(X, nbytes(a.N, a.h)) || !req(Wqkv_i) || !req_n(QKV_i, nbytes(a.N, a.qkv_cols)))
    return TP_MLP_ERR_INVALID_ARG;
  if (const tp_mlp_status ss = attn_ws_status(a, workspace, workspace_bytes, QKV_i, nbytes(a.N, a.qkv_cols)))
    return ss;
  const size_t wsu = attn_workspace(a);
  if (!spans_ok({{QKV_i, nbytes(a.N, a.qkv_cols)}, {wsu ? workspace : nullptr, wsu}},
                {{X, nbytes(a.N, a.h)}, {Wqkv_i, nbytes(a.h, a.qkv_cols)}}))
    return TP_MLP_ERR_INVALID_ARG;
  if (a.N == 0) return TP_MLP_OK;
  if (attn_small(a))
    return hip_status(skinny_product_launch((int)a.N, cu16(X), cu16(Wqkv_i), (int)a.h, (int)a.qkv_cols,
                                            attn_qkv_plan(a), static_cast<float*>(workspace), u16(QKV_i), stream));
  return hip_status(run_nn(a.N, a.qkv_cols, a.h, X, Wqkv_i, QKV_i, stream));
}

tp_mlp_status tp_attn_out_shard(const tp_attn_shape* s, const void* O_i, const void* Wo_i, void* Y_i,
                                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  AttnDims a;
  if (const tp_mlp_status ss = attn_status(s, a)) return ss;
  if (!req_n(O_i, nbytes(a.N, a.q_cols)) || !req(Wo_i) || !req_n(Y_i, nbytes(a.N, a.h))) return TP_MLP_ERR_INVALID_ARG;
  if (const tp_mlp_status ss = attn_ws_status(a, workspace, workspace_bytes, Y_i, nbytes(a.N, a.h))) return ss;
  const size_t wsu = attn_workspace(a);
  if (!spans_ok({{Y_i, nbytes(a.N, a.h)}, {wsu ? workspace : nullptr, wsu}},
                {{O_i, nbytes(a.N, a.q_cols)}, {Wo_i, nbytes(a.q_cols, a.h)}}))
    return TP_MLP_ERR_INVALID_ARG;
  if (a.N == 0) return TP_MLP_OK;
  if (attn_small(a))
    return hip_status(skinny_product_launch((int)a.N, cu16(O_i), cu16(Wo_i), (int)a.q_cols, (int)a.h,
                                            attn_out_plan(a), static_cast<float*>(workspace), u16(Y_i), stream));
  return hip_status(run_nn(a.N, a.h, a.q_cols, O_i, Wo_i, Y_i, stream));
}

tp_mlp_status tp_attn_out_bwd_shard(const tp_attn_shape* s, const void* dY, const void* O_i, const void* Wo_i,
                                    void* dO_i, float* dWo_i, hipStream_t stream) {
  AttnDims a;
  if (const tp_mlp_status ss = attn_status(s, a)) return ss;
  if (!req_n(dY, nbytes(a.N, a.h)) || !req_n(O_i, nbytes(a.N, a.q_cols)) || !req(Wo_i) ||
      !req_n(dO_i, nbytes(a.N, a.q_cols)) || !req(dWo_i))
    return TP_MLP_ERR_INVALID_ARG;
  if (!spans_ok({{dO_i, nbytes(a.N, a.q_cols)}, {dWo_i, (uint64_t)a.q_cols * a.h * 4}},
                {{dY, nbytes(a.N, a.h)}, {O_i, nbytes(a.N, a.q_cols)}, {Wo_i, nbytes(a.q_cols, a.h)}}))
    return TP_MLP_ERR_INVALID_ARG;
  if (a.N == 0) return hip_status(zero_f32_launch(dWo_i, a.q_cols * a.h, num_cu_current(), stream));
  // dWo_i is written after dO_i: until then its storage holds dO_i's k-split partials
  hipError_t e = run_nt(a.N, a.q_cols, a.h, dY, Wo_i, dO_i, stream, dWo_i, (uint64_t)a.q_cols * a.h, dO_cap(a));
  if (e == hipSuccess) e = run_tn(a.q_cols, a.h, a.N, O_i, dY, dWo_i, stream);
  return hip_status(e);
}

tp_mlp_status tp_attn_qkv_bwd_shard(const tp_attn_shape* s, const void* X, const void* Wqkv_i,
                                    const void* dQKV_i, float* dWqkv_i, void* dX_partial, hipStream_t stream) {
  AttnDims a;
  if (const tp_mlp_status ss = attn_status(s, a)) return ss;
  if (!req_n(X, nbytes(a.N, a.h)) || !req(Wqkv_i) || !req_n(dQKV_i, nbytes(a.N, a.qkv_cols)) || !req(dWqkv_i) ||
      !req_n(dX_partial, nbytes(a.N, a.h)))
    return TP_MLP_ERR_INVALID_ARG;
  if (!spans_ok({{dWqkv_i, (uint64_t)a.h * a.qkv_cols * 4}, {dX_partial, nbytes(a.N, a.h)}},
                {{X, nbytes(a.N, a.h)}, {Wqkv_i, nbytes(a.h, a.qkv_cols)}, {dQKV_i, nbytes(a.N, a.qkv_cols)}}))
    return TP_MLP_ERR_INVALID_ARG;
  if (a.N == 0) return hip_status(zero_f32_launch(dWqkv_i, a.h * a.qkv_cols, num_cu_current(), stream));
  // unmixed, dWqkv_i is written after dX_partial: until then its storage may hold the k-split partials
  return hip_status(run_attn_qkv_bwd(a, X, Wqkv_i, dQKV_i, dWqkv_i, dX_partial, nullptr, nullptr, nullptr,
                                     dWqkv_i, (uint64_t)a.h * a.qkv_cols, stream));
}

size_t tp_attn_out_dgrad_workspace_bytes(const tp_attn_shape* s) {
  AttnDims a;
  if (attn_status(s, a) != TP_MLP_OK || a.N == 0) return 0;
  return round256(attn_dO_part_floats(a) * sizeof(float));
}

tp_mlp_status tp_attn_out_dgrad_shard(const tp_attn_shape* s, const void* dY, const void* Wo_i, void* dO_i,
                                      void* workspace, size_t workspace_bytes, hipStream_t stream) {
  AttnDims a;
  if (const tp_mlp_status ss = attn_status(s, a)) return ss;
  if (!req_n(dY, nbytes(a.N, a.h)) || !req(Wo_i) || !req_n(dO_i, nbytes(a.N, a.q_cols)) || !opt_aligned(workspace))
    return TP_MLP_ERR_INVALID_ARG;
  const uint64_t pf = a.N > 0 ? attn_dO_part_floats(a) : 0;
  if (pf > 0 && (workspace == nullptr || workspace_bytes < pf * sizeof(float))) return TP_MLP_ERR_WORKSPACE;
  if (!spans_ok({{dO_i, nbytes(a.N, a.q_cols)}, {pf ? workspace : nullptr, pf * sizeof(float)}},
                {{dY, nbytes(a.N, a.h)}, {Wo_i, nbytes(a.q_cols, a.h)}}))
    return TP_MLP_ERR_INVALID_ARG;
  if (a.N == 0) return TP_MLP_OK;
  return hip_status(
      run_nt(a.N, a.q_cols, a.h, dY, Wo_i, dO_i, stream, static_cast<float*>(workspace), pf, dO_cap(a)));
}

tp_mlp_status tp_attn_qkv_bwd_out_wgrad_shard(const tp_attn_shape* s, const void* X, const void* Wqkv_i,
                                              const void* dQKV_i, const void* dY, const void* O_i, float* dWqkv_i,
                                              void* dX_partial, float* dWo_i, hipStream_t stream) {
  AttnDims a;
  if (const tp_mlp_status ss = attn_status(s, a)) return ss;
  if (!req_n(X, nbytes(a.N, a.h)) || !req(Wqkv_i) || !req_n(dQKV_i, nbytes(a.N, a.qkv_cols)) || !req(dWqkv_i) ||
      !req_n(dX_partial, nbytes(a.N, a.h)) || !req_n(dY, nbytes(a.N, a.h)) || !req_n(O_i, nbytes(a.N, a.q_cols)) ||
      !req(dWo_i))
    return TP_MLP_ERR_INVALID_ARG;
  if (!spans_ok({{dWqkv_i, (uint64_t)a.h * a.qkv_cols * 4}, {dX_partial, nbytes(a.N, a.h)},
                 {dWo_i, (uint64_t)a.q_cols * a.h * 4}},
                {{X, nbytes(a.N, a.h)}, {Wqkv_i, nbytes(a.h, a.qkv_cols)}, {dQKV_i, nbytes(a.N, a.qkv_cols)},
                 {dY, nbytes(a.N, a.h)}, {O_i, nbytes(a.N, a.q_cols)}}))
    return TP_MLP_ERR_INVALID_ARG;
  if (a.N == 0) {
    hipError_t e = zero_f32_launch(dWqkv_i, a.h * a.qkv_cols, num_cu_current(), stream);
    if (e == hipSuccess) e = zero_f32_launch(dWo_i, a.q_cols * a.h, num_cu_current(), stream);
    return hip_status(e);
  }
  return hip_status(run_attn_qkv_bwd(a, X, Wqkv_i, dQKV_i, dWqkv_i, dX_partial, dY, O_i, dWo_i, dWqkv_i,
                                     (uint64_t)a.h * a.qkv_cols, stream));
}

tp_mlp_status tp_sp_layernorm_fwd(int64_t rows, int64_t cols, float eps, const void* x, const void* gamma,
                                  const void* beta, void* y, float* mean, float* rstd, hipStream_t stream) {
  if (const tp_mlp_status ss = ln_status(rows, cols, eps, gamma, beta)) return ss;
  const uint64_t nb = (uint64_t)rows * (uint64_t)cols * 2;
  if (!req_n(x, nb) || !req_n(y, nb)) return TP_MLP_ERR_INVALID_ARG;
  if (!same_or_disjoint(y, nb, x, nb) || !disjoint(y, nb, gamma, (uint64_t)cols * 2) ||
      (beta && !disjoint(y, nb, beta, (uint64_t)cols * 2)) || !stash_ok(mean, rstd, rows, y, nb) ||
      (mean && (!disjoint(mean, (uint64_t)rows * 4, x, nb) || !disjoint(rstd, (uint64_t)rows * 4, x, nb))))
    return TP_MLP_ERR_INVALID_ARG;
  if (rows == 0) return TP_MLP_OK;
  return hip_status(ln_fwd_launch(cu16(x), rows, cols, eps, cu16(gamma), cu16(beta), u16(y), mean, rstd, stream));
}

tp_mlp_status tp_sp_reduce_scatter_layernorm_local(int32_t t, const void* const* partials, int64_t rows,
                                                   int64_t cols, int32_t rank, const void* bias,
                                                   const void* residual, void* z, float eps, const void* gamma,
                                                   const void* beta, void* y, float* mean, float* rstd,
                                                   hipStream_t stream) {
  PartialPtrs pp = {};
  if (const tp_mlp_status ss = rs_status(t, partials, rows, cols, rank, bias, residual, z, pp)) return ss;
  const int64_t shard = rows / t;
  if (const tp_mlp_status ss = ln_status(shard, cols, eps, gamma, beta)) return ss;
  const uint64_t nb = (uint64_t)shard * (uint64_t)cols * 2, full = (uint64_t)rows * (uint64_t)cols * 2;
  if (!req_n(y, nb)) return TP_MLP_ERR_INVALID_ARG;
  for (int r = 0; r < t; ++r)
    if (!disjoint(y, nb, pp.p[r], full)) return TP_MLP_ERR_INVALID_ARG;
  if (!disjoint(z, nb, gamma, (uint64_t)cols * 2) || (beta && !disjoint(z, nb, beta, (uint64_t)cols * 2)))
    return TP_MLP_ERR_INVALID_ARG;
  if (!disjoint(y, nb, z, nb) || (residual && !disjoint(y, nb, residual, nb)) ||
      (bias && !disjoint(y, nb, bias, (uint64_t)cols * 2)) || !disjoint(y, nb, gamma, (uint64_t)cols * 2) ||
      (beta && !disjoint(y, nb, beta, (uint64_t)cols * 2)) || !stash_ok(mean, rstd, shard, y, nb) ||
      (mean && (!disjoint(mean, (uint64_t)shard * 4, z, nb) || !disjoint(rstd, (uint64_t)shard * 4, z, nb))))
    return TP_MLP_ERR_INVALID_ARG;
  if (shard == 0) return TP_MLP_OK;
  return hip_status(ln_fwd_fused_launch(pp, t, shard, cols, (int64_t)rank * shard, cu16(bias), cu16(residual),
                                        u16(z), eps, cu16(gamma), cu16(beta), u16(y), mean, rstd, stream));
}

size_t tp_sp_layernorm_bwd_workspace_bytes(int64_t rows, int64_t cols) {
  if (rows < 1 || rows >= (int64_t)1 << 31 || cols < 8 || cols % 8 != 0 || cols > LN_MAX_COLS) return 0;
  return ln_bwd_workspace_bytes(rows, cols);
}

tp_mlp_status tp_sp_layernorm_bwd(int64_t rows, int64_t cols, const void* x, const void* gamma, const float* mean,
                                  const float* rstd, const void* dy, const void* dres, void* dx, float* dgamma,
                                  float* dbeta, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (const tp_mlp_status ss = ln_status(rows, cols, 1.0f, gamma, nullptr)) return ss;
  const uint64_t nb = (uint64_t)rows * (uint64_t)cols * 2, gb = (uint64_t)cols * 4, sb = (uint64_t)rows * 4;
  if (!req_n(x, nb) || !req_n(mean, sb) || !req_n(rstd, sb) || !req_n(dy, nb) || !opt_aligned(dres) ||
      !req_n(dx, nb) || !req(dgamma) || !opt_aligned(dbeta))
    return TP_MLP_ERR_INVALID_ARG;
  const size_t need = ln_bwd_workspace_bytes(rows, cols);
  if (!disjoint(dx, nb, x, nb) || !same_or_disjoint(dx, nb, dy, nb) || (dres && !same_or_disjoint(dx, nb, dres, nb)) ||
      !disjoint(dx, nb, gamma, (uint64_t)cols * 2) || !disjoint(dx, nb, mean, (uint64_t)rows * 4) ||
      !disjoint(dx, nb, rstd, (uint64_t)rows * 4))
    return TP_MLP_ERR_INVALID_ARG;
  // dgamma and dbeta: disjoint from every input, dx and each other
  const float* grads[2] = {dgamma, dbeta};
  for (const float* g : grads) {
    if (!g) continue;
    if (!disjoint(g, gb, dx, nb) || !disjoint(g, gb, x, nb) || !disjoint(g, gb, dy, nb) ||
        (dres && !disjoint(g, gb, dres, nb)) || !disjoint(g, gb, gamma, (uint64_t)cols * 2) ||
        !disjoint(g, gb, mean, (uint64_t)rows * 4) || !disjoint(g, gb, rstd, (uint64_t)rows * 4))
      return TP_MLP_ERR_INVALID_ARG;
  }
  if (dbeta && !disjoint(dbeta, gb, dgamma, gb)) return TP_MLP_ERR_INVALID_ARG;
  if (rows == 0) {  // dgamma and dbeta are sums over no rows
    hipError_t e = zero_f32_launch(dgamma, cols, num_cu_current(), stream);
    if (e == hipSuccess) e = zero_f32_launch(dbeta, cols, num_cu_current(), stream);
    return hip_status(e);
  }
  if (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)) return TP_MLP_ERR_WORKSPACE;
  if (!disjoint(workspace, need, dx, nb) || !disjoint(workspace, need, dgamma, gb) ||
      (dbeta && !disjoint(workspace, need, dbeta, gb)) || !disjoint(workspace, need, x, nb) ||
      !disjoint(workspace, need, dy, nb) || (dres && !disjoint(workspace, need, dres, nb)) ||
      !disjoint(workspace, need, gamma, (uint64_t)cols * 2) || !disjoint(workspace, need, mean, (uint64_t)rows * 4) ||
      !disjoint(workspace, need, rstd, (uint64_t)rows * 4))
    return TP_MLP_ERR_INVALID_ARG;
  return hip_status(ln_bwd_launch(cu16(x), cu16(gamma), mean, rstd, cu16(dy), cu16(dres), u16(dx), rows, cols,
                                  dgamma, dbeta, static_cast<float*>(workspace), stream));
}

tp_mlp_status tp_sp_sum_grads_local(int32_t t, const float* const* grads, int64_t n, float* out,
                                    hipStream_t stream) {
  if (grads == nullptr || t < 1) return TP_MLP_ERR_INVALID_ARG;
  if (t > MAX_T) return TP_MLP_ERR_UNSUPPORTED;
  if (n < 0 || n % 4 != 0 || n > (int64_t)1 << 40) return TP_MLP_ERR_INVALID_ARG;
  const uint64_t nb = (uint64_t)n * 4;
  if (!req_n(out, nb)) return TP_MLP_ERR_INVALID_ARG;
  GradPtrs g = {};
  for (int r = 0; r < t; ++r) {
    if (!req_n(grads[r], nb)) return TP_MLP_ERR_INVALID_ARG;
    if (r == 0 ? !same_or_disjoint(out, nb, grads[r], nb) : !disjoint(out, nb, grads[r], nb))
      return TP_MLP_ERR_INVALID_ARG;
    g.p[r] = grads[r];
  }
  if (n == 0) return TP_MLP_OK;
  return hip_status(sum_f32_launch(g, t, n, out, stream));
}

}  // extern "C"

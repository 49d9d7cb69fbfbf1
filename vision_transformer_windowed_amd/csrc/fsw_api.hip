// C ABI of the window-attention library: argument validation, workspace sizing, dispatch.
//
// Every check runs on the host before any HIP call, so an invalid call never touches the device.
// Dispatch: bf16 with d == 32 and M <= 32 goes to the MFMA kernels; everything else (float32
// tensors, other d) goes to the float32-arithmetic kernels.
#include <algorithm>

#include "../../include/flashswin.h"
#include "fsw_launch.h"

namespace {

constexpr int kMaxM = 32;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool supported_d(int d) { return d == 8 || d == 16 || d == 32 || d == 64; }

// Shape rules shared by forward, backward and workspace sizing.  Fills g on success.
int check_shape(int64_t B, int64_t Hg, int64_t Wg, int heads, int d, int M, int shift, int dtype, fsw::Geom* g) {
  if (B < 0 || Hg < 1 || Wg < 1 || heads < 1 || M < 1 || d < 1) return FSW_ERR_INVALID_ARG;
  if (Hg % M != 0 || Wg % M != 0) return FSW_ERR_INVALID_ARG;
  if (shift < 0 || shift >= M) return FSW_ERR_INVALID_ARG;
  if (d % 4 != 0) return FSW_ERR_INVALID_ARG;
  if (dtype != FSW_F32 && dtype != FSW_BF16) return FSW_ERR_INVALID_ARG;
  if (!supported_d(d) || M > kMaxM) return FSW_ERR_UNSUPPORTED;
  // int32 grid coordinates and int64 element offsets: keep every product well inside int64,
  // and the flat 1-D launch grid inside 2^31 workgroups.
  const int64_t lim = (int64_t)1 << 30;
  if (Hg > lim || Wg > lim || heads > (1 << 20)) return FSW_ERR_UNSUPPORTED;
  const long double elems = (long double)B * Hg * Wg * heads * d;
  if (elems > (long double)((int64_t)1 << 56)) return FSW_ERR_UNSUPPORTED;
  const long double wgs = (long double)B * (Hg / M) * (Wg / M) * heads * 8;
  if (wgs > (long double)((int64_t)1 << 31) - 1) return FSW_ERR_UNSUPPORTED;
  g->B = B;
  g->Hg = (int)Hg;
  g->Wg = (int)Wg;
  g->heads = heads;
  g->d = d;
  g->M = M;
  g->shift = shift;
  g->nH = (int)(Hg / M);
  g->nW = (int)(Wg / M);
  g->N = M * M;
  g->xs = (int64_t)heads * d;
  g->os = (int64_t)heads * d;
  return FSW_OK;
}

size_t elem_bytes(int dtype) { return dtype == FSW_BF16 ? 2 : 4; }

// Byte ranges [a, a + na) and [b, b + nb) overlap (a null or empty range overlaps nothing).
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// A buffer and its size in bytes.
struct Span {
  const void* p;
  size_t n;
};
// Every output span is disjoint from every input span and from the other outputs.  Inputs may
// share memory with each other (they are only read).
template <size_t NO, size_t NI>
bool outputs_disjoint(const Span (&outs)[NO], const Span (&ins)[NI]) {
  for (size_t i = 0; i < NO; ++i) {
    for (size_t j = 0; j < NI; ++j)
      if (overlap(outs[i].p, outs[i].n, ins[j].p, ins[j].n)) return false;
    for (size_t j = i + 1; j < NO; ++j)
      if (overlap(outs[i].p, outs[i].n, outs[j].p, outs[j].n)) return false;
  }
  return true;
}

// Bytes of one token-grid tensor, of LSE and of one theta table of geometry g.
struct Sizes {
  size_t tens, lse, theta;
};
Sizes sizes_of(const fsw::Geom& g, int dtype) {
  const size_t tokens = (size_t)(g.B * g.Hg * g.Wg);
  return {tokens * (size_t)g.os * elem_bytes(dtype), tokens * (size_t)g.heads * 4,
          (size_t)g.heads * (size_t)(g.d / 4) * 4};
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct WsLayout {
  size_t delta_off, scal_off, partials_off, total;
  int64_t n_partials;
};

WsLayout workspace_layout(const fsw::Geom& g, bool mfma) {
  WsLayout w;
  const int64_t rows = g.B * g.Hg * g.Wg * g.heads;
  const int64_t nwh = g.B * g.nH * g.nW * g.heads;
  w.delta_off = 0;
  w.scal_off = align256((size_t)rows * sizeof(float));
  w.partials_off = w.scal_off + align256((size_t)nwh * 4 * sizeof(float));
  w.n_partials = mfma ? fsw::bwd_mfma_partials(g) : fsw::bwd_scalar_partials(g);
  w.total = w.partials_off + align256((size_t)w.n_partials * (g.d / 2) * sizeof(float));
  return w;
}

bool use_mfma_fwd(const fsw::Geom& g, int dtype) { return dtype == FSW_BF16 && g.d == 32 && g.M <= kMaxM; }
bool use_mfma(const fsw::Geom& g, int dtype) { return fsw::kHaveMfmaBwd && use_mfma_fwd(g, dtype); }

// Pointer checks and dispatch of a forward whose shape (and q/k/v token stride) is in g.
int fwd_impl(const void* q, const void* k, const void* v, const float* theta_row, const float* theta_col, void* out,
             float* lse, const fsw::Geom& g, int dtype, void* hip_stream) {
  if (!q || !k || !v || !out || !theta_row || !theta_col) return FSW_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16)) return FSW_ERR_INVALID_ARG;
  if (!aligned(theta_row, 4) || !aligned(theta_col, 4) || (lse && !aligned(lse, 4))) return FSW_ERR_INVALID_ARG;
  fsw::FwdArgs a{q, k, v, theta_row, theta_col, out, lse, g, dtype};
  hipStream_t s = reinterpret_cast<hipStream_t>(hip_stream);
  const hipError_t e = use_mfma_fwd(g, dtype) ? fsw::launch_fwd_mfma(a, s) : fsw::launch_fwd_scalar(a, s);
  return e == hipSuccess ? FSW_OK : FSW_ERR_HIP;
}

// Pointer, workspace checks and dispatch of a backward whose shape (and strides) is in g.
int bwd_impl(const void* q, const void* k, const void* v, const void* out, const void* dout, const float* lse,
             const float* theta_row, const float* theta_col, void* dq, void* dk, void* dv, float* dtheta_row,
             float* dtheta_col, void* workspace, size_t workspace_bytes, const fsw::Geom& g, int dtype,
             void* hip_stream) {
  const void* ptrs16[] = {q, k, v, out, dout, dq, dk, dv};
  for (const void* p : ptrs16)
    if (!p || !aligned(p, 16)) return FSW_ERR_INVALID_ARG;
  const void* ptrs4[] = {lse, theta_row, theta_col, dtheta_row, dtheta_col};
  for (const void* p : ptrs4)
    if (!p || !aligned(p, 4)) return FSW_ERR_INVALID_ARG;
  if (dtheta_row == dtheta_col) return FSW_ERR_INVALID_ARG;
  const bool mfma = use_mfma(g, dtype);
  const WsLayout ws = workspace_layout(g, mfma);
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < ws.total) return FSW_ERR_WORKSPACE;
  char* base = static_cast<char*>(workspace);
  fsw::BwdArgs a{q,  k,  v,          out,        dout, lse, theta_row, theta_col,
                 dq, dk, dv,         dtheta_row, dtheta_col, g, dtype,
                 reinterpret_cast<float*>(base + ws.delta_off), reinterpret_cast<float*>(base + ws.scal_off),
                 reinterpret_cast<float*>(base + ws.partials_off), ws.n_partials};
  hipStream_t s = reinterpret_cast<hipStream_t>(hip_stream);
  const hipError_t e = mfma ? fsw::launch_bwd_mfma(a, s) : fsw::launch_bwd_scalar(a, s);
  return e == hipSuccess ? FSW_OK : FSW_ERR_HIP;
}

}  // namespace

extern "C" {

int flashswin_version(void) { return 101; }

const char* flashswin_status_string(int status) {
  switch (status) {
    case FSW_OK: return "FSW_OK";
    case FSW_ERR_INVALID_ARG: return "FSW_ERR_INVALID_ARG: invalid shape, pointer, alignment, shift or dtype";
    case FSW_ERR_UNSUPPORTED: return "FSW_ERR_UNSUPPORTED: valid arguments this library does not implement";
    case FSW_ERR_WORKSPACE: return "FSW_ERR_WORKSPACE: workspace missing or too small";
    case FSW_ERR_HIP: return "FSW_ERR_HIP: a HIP kernel launch failed";
    default: return "unknown flashswin status";
  }
}

int flashswin_wattn_fwd(const void* q, const void* k, const void* v, const float* theta_row, const float* theta_col,
                        void* out, float* lse, int64_t B, int64_t Hg, int64_t Wg, int heads, int d, int M, int shift,
                        int dtype, void* hip_stream) {
  fsw::Geom g;
  int st = check_shape(B, Hg, Wg, heads, d, M, shift, dtype, &g);
  if (st != FSW_OK) return st;
  if (B == 0) return FSW_OK;
  const Sizes z = sizes_of(g, dtype);
  const Span outs[] = {{out, z.tens}, {lse, z.lse}};
  const Span ins[] = {{q, z.tens}, {k, z.tens}, {v, z.tens}, {theta_row, z.theta}, {theta_col, z.theta}};
  if (!outputs_disjoint(outs, ins)) return FSW_ERR_INVALID_ARG;
  return fwd_impl(q, k, v, theta_row, theta_col, out, lse, g, dtype, hip_stream);
}

int flashswin_wattn_fwd_packed(const void* qkv, const float* theta_row, const float* theta_col, void* out, float* lse,
                               int64_t B, int64_t Hg, int64_t Wg, int heads, int d, int M, int shift, int dtype,
                               void* hip_stream) {
  fsw::Geom g;
  int st = check_shape(B, Hg, Wg, heads, d, M, shift, dtype, &g);
  if (st != FSW_OK) return st;
  if (B == 0) return FSW_OK;
  if ((long double)B * Hg * Wg * 3 * heads * d > (long double)((int64_t)1 << 56)) return FSW_ERR_UNSUPPORTED;
  if (!qkv) return FSW_ERR_INVALID_ARG;
  const size_t eb = elem_bytes(dtype);
  const Sizes z = sizes_of(g, dtype);
  const Span outs[] = {{out, z.tens}, {lse, z.lse}};
  const Span ins[] = {{qkv, 3 * z.tens}, {theta_row, z.theta}, {theta_col, z.theta}};
  if (!outputs_disjoint(outs, ins)) return FSW_ERR_INVALID_ARG;
  g.xs = 3 * g.os;
  const char* base = static_cast<const char*>(qkv);
  const size_t slot = (size_t)g.os * eb;  // bytes from q to k and from k to v within a token
  return fwd_impl(base, base + slot, base + 2 * slot, theta_row, theta_col, out, lse, g, dtype, hip_stream);
}

size_t flashswin_wattn_bwd_workspace_size(int64_t B, int64_t Hg, int64_t Wg, int heads, int d, int M, int shift,
                                          int dtype) {
  fsw::Geom g;
  if (check_shape(B, Hg, Wg, heads, d, M, shift, dtype, &g) != FSW_OK) return 0;
  if (B == 0) return 0;
  return workspace_layout(g, use_mfma(g, dtype)).total;
}

int flashswin_wattn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
                        const float* lse, const float* theta_row, const float* theta_col, void* dq, void* dk, void* dv,
                        float* dtheta_row, float* dtheta_col, void* workspace, size_t workspace_bytes, int64_t B,
                        int64_t Hg, int64_t Wg, int heads, int d, int M, int shift, int dtype, void* hip_stream) {
  fsw::Geom g;
  int st = check_shape(B, Hg, Wg, heads, d, M, shift, dtype, &g);
  if (st != FSW_OK) return st;
  if (B == 0) return FSW_OK;
  const Sizes z = sizes_of(g, dtype);
  const Span outs[] = {{dq, z.tens},         {dk, z.tens},          {dv, z.tens},
                       {dtheta_row, z.theta}, {dtheta_col, z.theta}, {workspace, workspace_bytes}};
  const Span ins[] = {{q, z.tens},   {k, z.tens},           {v, z.tens},          {out, z.tens},
                      {dout, z.tens}, {lse, z.lse}, {theta_row, z.theta}, {theta_col, z.theta}};
  if (!outputs_disjoint(outs, ins)) return FSW_ERR_INVALID_ARG;
  return bwd_impl(q, k, v, out, dout, lse, theta_row, theta_col, dq, dk, dv, dtheta_row, dtheta_col, workspace,
                  workspace_bytes, g, dtype, hip_stream);
}

int flashswin_wattn_bwd_packed(const void* qkv, const void* out, const void* dout, const float* lse,
                               const float* theta_row, const float* theta_col, void* dqkv, float* dtheta_row,
                               float* dtheta_col, void* workspace, size_t workspace_bytes, int64_t B, int64_t Hg,
                               int64_t Wg, int heads, int d, int M, int shift, int dtype, void* hip_stream) {
  fsw::Geom g;
  int st = check_shape(B, Hg, Wg, heads, d, M, shift, dtype, &g);
  if (st != FSW_OK) return st;
  if (B == 0) return FSW_OK;
  if ((long double)B * Hg * Wg * 3 * heads * d > (long double)((int64_t)1 << 56)) return FSW_ERR_UNSUPPORTED;
  if (!qkv || !dqkv) return FSW_ERR_INVALID_ARG;
  const size_t eb = elem_bytes(dtype);
  const Sizes z = sizes_of(g, dtype);
  const Span outs[] = {{dqkv, 3 * z.tens}, {dtheta_row, z.theta}, {dtheta_col, z.theta},
                       {workspace, workspace_bytes}};
  const Span ins[] = {{qkv, 3 * z.tens}, {out, z.tens}, {dout, z.tens}, {lse, z.lse}, {theta_row, z.theta},
                      {theta_col, z.theta}};
  if (!outputs_disjoint(outs, ins)) return FSW_ERR_INVALID_ARG;
  g.xs = 3 * g.os;
  const size_t slot = (size_t)g.os * eb;
  const char* x = static_cast<const char*>(qkv);
  char* dx = static_cast<char*>(dqkv);
  return bwd_impl(x, x + slot, x + 2 * slot, out, dout, lse, theta_row, theta_col, dx, dx + slot, dx + 2 * slot,
                  dtheta_row, dtheta_col, workspace, workspace_bytes, g, dtype, hip_stream);
}

}  // extern "C"

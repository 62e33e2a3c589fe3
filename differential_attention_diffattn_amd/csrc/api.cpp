// api.cpp -- the C ABI declared in include/diffattn.h: argument validation on
// the host, then dispatch to the gfx950 kernels.
//
// Validation makes no HIP call, so every error status is reachable (and
// tested) on a machine without a GPU; a call that fails validation enqueues
// nothing and leaves `out` untouched.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/diffattn.h"
#include "kernels.hpp"

namespace {

using da::TIn;
using da::TOut;

bool aligned(const void* p, uintptr_t n) { return ((uintptr_t)p % n) == 0; }

// A dense-row tensor (unit-stride head_dim, 128-bit rows): non-null, 16-byte
// aligned base, non-negative role strides that are multiples of `mult`
// elements.
da_status check_rows(const void* p, int64_t sb, int64_t sh, int64_t st, int64_t mult) {
  if (!p) return DA_E_NULL;
  if (!aligned(p, 16)) return DA_E_LAYOUT;
  const int64_t s[3] = {sb, sh, st};
  for (int64_t x : s)
    if (x < 0 || x % mult != 0) return DA_E_LAYOUT;
  return DA_OK;
}
da_status check_in(const da_in& t, int64_t mult) { return check_rows(t.ptr, t.sb, t.sh, t.st, mult); }
da_status check_out(const da_out& t, int64_t mult) { return check_rows(t.ptr, t.sb, t.sh, t.st, mult); }

// fp32 logits without a head_dim axis: only element alignment is needed.
da_status check_logits(const da_in& t) {
  if (!t.ptr) return DA_E_NULL;
  if (!aligned(t.ptr, 4)) return DA_E_LAYOUT;
  if (t.sb < 0 || t.sh < 0 || t.st < 0) return DA_E_LAYOUT;
  return DA_OK;
}

#define DA_TRY(x)                   \
  do {                              \
    const da_status _s = (x);       \
    if (_s != DA_OK) return _s;     \
  } while (0)

TIn tin(const da_in& t) { return TIn{t.ptr, t.sb, t.sh, t.st}; }
TOut tout(const da_out& t) { return TOut{t.ptr, t.sb, t.sh, t.st}; }

float log2e_over_sqrt(int d) { return (float)(1.4426950408889634 / sqrt((double)d)); }

// Rotary embedding: theta must be a finite number > 0; positions stay below
// 2^24 (exact in fp32).
bool rope_theta_ok(float theta) { return theta > 0.f && theta < INFINITY; }
// w_c = theta^(-2c/d) for c < d/2, as hi + lo floats (d <= 256).
void rope_tab(float theta, int d, da::RopeTab* t) {
  for (int c = 0; c < 128; ++c) {
    const double w = c < d / 2 ? pow((double)theta, -2.0 * c / (double)d) : 0.0;
    t->hi[c] = (float)w;
    t->lo[c] = (float)(w - (double)t->hi[c]);
  }
}
constexpr long long kMaxRopePos = 1LL << 24;

// The library's own rotated-k buffer inside a caller workspace: [B,T,H,d]
// contiguous bf16.
struct RopeK {
  float theta;
  void* ws;
  size_t ws_bytes;
};
size_t rope_k_bytes(int B, int T, int H, int d) { return ((size_t)B * T * H * d * 2 + 255) / 256 * 256; }

da_status launch_status(hipError_t e) { return e == hipSuccess ? DA_OK : DA_E_LAUNCH; }

// Largest grid the launchers build, for the overflow check.
bool grid_fits(long long n) { return n >= 1 && n <= 0x7fffffffLL; }

// The prefill kernels address a 128-key tile with 32-bit byte offsets from a
// per-tile base, which bounds the key/value token stride.
constexpr int64_t kMaxTokenStride = int64_t(1) << 24;  // elements

da_status validate_v2_common(int dtype, int B, int T, int Hq, int Hkv, int d) {
  if (dtype != DA_FP32 && dtype != DA_BF16) return DA_E_DTYPE;
  if (B < 1 || T < 1 || Hq < 1 || Hkv < 1 || d < 1) return DA_E_SHAPE;
  if (Hq % Hkv != 0 || (Hq / Hkv) % 2 != 0) return DA_E_SHAPE;
  if (dtype != DA_BF16) return DA_E_UNSUPPORTED;
  if (d != 64 && d != 128) return DA_E_UNSUPPORTED;
  return DA_OK;
}

// Split geometry of a decode call: nq query tokens x G heads form the
// columns a workgroup scores 16 or 32 at a time (column groups); the cache is
// split along its length for B x column groups x Hkv units.
struct DecodeGeom {
  int ncg;
  da::DecodeSplit sp;
};
DecodeGeom decode_geom(int B, int L, int nq, int Hq, int Hkv, int max_chunk, int max_splits = 0x7fffffff) {
  DecodeGeom r;
  r.ncg = da::decode_column_groups(nq, Hq / Hkv);
  r.sp = da::decode_split(B * r.ncg, L, Hkv, max_chunk, max_splits);
  return r;
}
bool decode_sizes_ok(int B, int L, int nq, int Hq, int Hkv, int d) {
  if (B < 1 || L < 1 || nq < 1 || Hq < 1 || Hkv < 1 || d < 1) return false;
  if (Hq % Hkv != 0 || (Hq / Hkv) % 2 != 0) return false;
  return (long long)B * nq <= 0x7fffffffLL && (long long)nq * Hq <= 0x7fffffffLL;
}
// Bytes of one split's partials: (m, l, O[d]) fp32 per (b, kv head, column).
size_t decode_split_bytes(int B, int nq, int Hq, int Hkv, int d) {
  return (size_t)B * Hkv * (size_t)nq * (size_t)(Hq / Hkv) * (size_t)(d + 2) * sizeof(float);
}
size_t decode_ws_bytes(int B, int L, int nq, int Hq, int Hkv, int d, int max_chunk, int max_splits = 0x7fffffff) {
  if (!decode_sizes_ok(B, L, nq, Hq, Hkv, d)) return 0;
  const DecodeGeom gm = decode_geom(B, L, nq, Hq, Hkv, max_chunk, max_splits);
  return gm.sp.nsplit * decode_split_bytes(B, nq, Hq, Hkv, d);
}

// ---- the decode entry point that allocates nothing --------------------------
// Its split partials live in this file-scope device array: one copy per GPU,
// allocated when the library's code object is loaded and held until the
// process ends.  kScratchBytes bounds the partials (B x Hkv x splits x
// columns x (d + 2) fp32); the split count is lowered until they fit.
constexpr size_t kScratchBytes = size_t(16) << 20;
constexpr int kMaxDevices = 64;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of `scratch` on the current device.  In host code the
// array's name is only a stand-in: its device address is looked up once per
// device, with that device current, and kept.
void* scratch_on_current_device() {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    addr[dev] = p;
  }
  return addr[dev];
}

// Shared by the dense and paged decode entry points.  q, lam and out carry a
// token axis (stride st) only when nq > 1.  Paged: k / v are page pools and
// `pg` describes the table; dense: pg.block_table is null.
struct PagedArgs {
  int num_pages, page_size;
  const int32_t* block_table;
  int64_t bt_stride;
  const int32_t* seq_lens;
};
da_status decode_impl(int softmax1, int dtype, int B, int L, int nq, int Hq, int Hkv, int d, da_in q,
                      da_in kc, da_in vc, const PagedArgs* pg, da_in lam, da_out out, void* workspace,
                      size_t workspace_bytes, void* stream, float rope_theta = 0.f,
                      int max_splits = 0x7fffffff, bool use_scratch = false) {
  if (dtype != DA_FP32 && dtype != DA_BF16) return DA_E_DTYPE;
  if (rope_theta != 0.f && (!rope_theta_ok(rope_theta) || (long long)L >= kMaxRopePos)) return DA_E_SHAPE;
  if (!decode_sizes_ok(B, L, nq, Hq, Hkv, d)) return DA_E_SHAPE;
  if (!pg && nq > L) return DA_E_SHAPE;  // the new tokens are the last nq cache entries
  const int page_size = pg ? pg->page_size : 0;
  if (pg) {
    if (pg->num_pages < 1) return DA_E_SHAPE;
    if (page_size < 16 || page_size > (1 << 30) || (page_size & (page_size - 1)) != 0) return DA_E_SHAPE;
    if (pg->bt_stride < ((int64_t)L + page_size - 1) / page_size) return DA_E_SHAPE;
  }
  const int64_t mult = dtype == DA_BF16 ? 8 : 4;
  const int64_t qst = nq > 1 ? q.st : 0, ost = nq > 1 ? out.st : 0;
  DA_TRY(check_rows(q.ptr, q.sb, q.sh, qst, mult));
  DA_TRY(check_in(kc, mult));
  DA_TRY(check_in(vc, mult));
  if (pg) {
    if (!pg->block_table || !pg->seq_lens) return DA_E_NULL;
    if (!aligned(pg->block_table, 4) || !aligned(pg->seq_lens, 4)) return DA_E_LAYOUT;
  }
  da_in lam2 = lam;
  lam2.st = nq > 1 ? lam.st : 0;
  DA_TRY(check_logits(lam2));
  DA_TRY(check_rows(out.ptr, out.sb, out.sh, ost, mult));
  DA_TRY(validate_v2_common(dtype, B, L, Hq, Hkv, d));
  if (Hq / Hkv > 16) return DA_E_UNSUPPORTED;  // one 16-wide MFMA column block per head group
  if (pg) {  // the kernel addresses a row within a page with a 32-bit element offset
    if ((int64_t)page_size * kc.st >= (int64_t(1) << 31) || (int64_t)page_size * vc.st >= (int64_t(1) << 31))
      return DA_E_UNSUPPORTED;
  } else if (kc.st >= kMaxTokenStride || vc.st >= kMaxTokenStride) {
    return DA_E_UNSUPPORTED;  // rows of a 32-token block are addressed with 32-bit byte offsets
  }
  const int max_chunk = pg ? da::kPagedMaxChunk : da::kDenseMaxChunk;
  const size_t need = decode_ws_bytes(B, L, nq, Hq, Hkv, d, max_chunk, max_splits);
  if (use_scratch) {  // every argument checked: now the static scratch of this device
    if (need > kScratchBytes) return DA_E_SCRATCH;
    workspace = scratch_on_current_device();
    workspace_bytes = kScratchBytes;
    if (!workspace) return DA_E_LAUNCH;
  }
  if (!workspace || !aligned(workspace, 16) || workspace_bytes < need) return DA_E_WORKSPACE;
  const DecodeGeom gm = decode_geom(B, L, nq, Hq, Hkv, max_chunk, max_splits);
  if (!grid_fits(da::decode_split_grid(B * gm.ncg, Hkv, gm.sp.nsplit)) || !grid_fits((long long)B * nq * (Hq / 2)))
    return DA_E_SHAPE;

  da::DecodeArgs a{};
  a.q = TIn{q.ptr, q.sb, q.sh, qst};
  a.k = tin(kc);
  a.v = tin(vc);
  a.lam = TIn{lam.ptr, lam.sb, lam.sh, lam2.st};
  a.out = TOut{out.ptr, out.sb, out.sh, ost};
  a.ws = (float*)workspace;
  a.sl2 = log2e_over_sqrt(d);
  a.B = B, a.L = L, a.Hq = Hq, a.Hkv = Hkv, a.G = Hq / Hkv;
  a.chunk = gm.sp.chunk;
  a.nsplit = gm.sp.nsplit;
  a.nq = nq;
  a.ncg = gm.ncg;
  a.softmax1 = softmax1;
  if (rope_theta != 0.f) {
    a.rope = 1;
    rope_tab(rope_theta, d, &a.rope_w);
  }
  if (pg) {
    a.block_table = pg->block_table;
    a.bt_stride = pg->bt_stride;
    a.seq_lens = pg->seq_lens;
    int shift = 0;
    while ((1 << shift) < page_size) ++shift;
    a.page_shift = shift;
    a.page_mask = page_size - 1;
    a.num_pages = pg->num_pages;
  }
  return launch_status(da::launch_decode_bf16(d, a, (hipStream_t)stream));
}

}  // namespace

extern "C" {

double diffattn_lambda_init(int layer_index) { return 0.8 - 0.6 * exp(-0.3 * (double)layer_index); }

const char* diffattn_status_string(da_status s) {
  switch (s) {
    case DA_OK: return "ok";
    case DA_E_NULL: return "a required pointer is NULL";
    case DA_E_DTYPE: return "unknown dtype";
    case DA_E_SHAPE: return "a size is < 1 or sizes are inconsistent";
    case DA_E_LAYOUT: return "misaligned pointer or invalid stride";
    case DA_E_UNSUPPORTED: return "no kernel for these (valid) arguments";
    case DA_E_WORKSPACE: return "decode workspace missing, misaligned or too small";
    case DA_E_LAUNCH: return "the HIP runtime rejected a kernel launch";
    case DA_E_SCRATCH: return "sizes need more than the library's static decode scratch";
  }
  return "unknown status";
}

static da_status v1_fwd_impl(int softmax1, int dtype, int B, int H, int T, int d, da_in q1, da_in q2,
                             da_in k1, da_in k2,
                          da_in v, const float* lam_q1, const float* lam_k1, const float* lam_q2,
                          const float* lam_k2, int layer_index, da_out out, void* stream,
                          const da_out* attn1 = nullptr, const da_out* attn2 = nullptr, float* lse = nullptr,
                          const RopeK* rope = nullptr) {
  if (dtype != DA_FP32 && dtype != DA_BF16) return DA_E_DTYPE;
  if (B < 1 || H < 1 || T < 1 || d < 1 || layer_index < 0) return DA_E_SHAPE;
  if (rope && (!rope_theta_ok(rope->theta) || (long long)T >= kMaxRopePos)) return DA_E_SHAPE;
  const int64_t mult = dtype == DA_BF16 ? 8 : 4;
  DA_TRY(check_in(q1, mult));
  DA_TRY(check_in(q2, mult));
  DA_TRY(check_in(k1, mult));
  DA_TRY(check_in(k2, mult));
  DA_TRY(check_in(v, mult));
  DA_TRY(check_out(out, mult));
  if (!lam_q1 || !lam_k1 || !lam_q2 || !lam_k2) return DA_E_NULL;
  if (!aligned(lam_q1, 4) || !aligned(lam_k1, 4) || !aligned(lam_q2, 4) || !aligned(lam_k2, 4))
    return DA_E_LAYOUT;
  if (dtype == DA_BF16 && d != 64 && d != 128) return DA_E_UNSUPPORTED;
  if (dtype == DA_FP32 && d != 32 && d != 64 && d != 128) return DA_E_UNSUPPORTED;
  if (dtype == DA_BF16 && (k1.st >= kMaxTokenStride || k2.st >= kMaxTokenStride || v.st >= kMaxTokenStride))
    return DA_E_UNSUPPORTED;
  if (!grid_fits((long long)B * H * ((T + 31) / 32))) return DA_E_SHAPE;
  if (attn1) {  // training forward (bf16 only)
    if (dtype != DA_BF16) return DA_E_UNSUPPORTED;
    DA_TRY(check_out(*attn1, 8));
    DA_TRY(check_out(*attn2, 8));
    if (!lse) return DA_E_NULL;
    if (!aligned(lse, 4)) return DA_E_LAYOUT;
  }

  if (rope) {
    if (dtype != DA_BF16) return DA_E_UNSUPPORTED;
    const size_t kb = rope_k_bytes(B, T, H, d);
    if (!rope->ws || !aligned(rope->ws, 256) || rope->ws_bytes < 2 * kb) return DA_E_WORKSPACE;
  }

  const float li = (float)diffattn_lambda_init(layer_index);
  hipStream_t s = (hipStream_t)stream;
  if (dtype == DA_BF16) {
    const da_in k1o = k1, k2o = k2;
    if (rope) {  // k1, k2 rotated into the workspace as [B,H,T,d]; q1, q2 in the kernel's prologue
      for (int m = 0; m < 2; ++m) {
        da::RopeArgs r{};
        r.x = tin(m ? k2 : k1);
        char* dst = (char*)rope->ws + m * rope_k_bytes(B, T, H, d);
        r.out = TOut{dst, (int64_t)H * T * d, (int64_t)T * d, (int64_t)d};
        r.B = B, r.T = T, r.H = H, r.d = d, r.pos0 = 0;
        rope_tab(rope->theta, d, &r.w);
        const da_status st = launch_status(da::launch_rope_bf16(r, s));
        if (st != DA_OK) return st;
        (m ? k2 : k1) = da_in{dst, (int64_t)H * T * d, (int64_t)T * d, (int64_t)d};
      }
    }
    da::PrefillArgs a{};
    a.q1 = tin(q1), a.q2 = tin(q2), a.k1 = tin(k1), a.k2 = tin(k2), a.v = tin(v);
    a.k1o = tin(k1o), a.k2o = tin(k2o);
    if (rope) {
      a.rope = 1;
      rope_tab(rope->theta, d, &a.rope_w);
    }
    a.out = tout(out);
    a.lq1 = lam_q1, a.lk1 = lam_k1, a.lq2 = lam_q2, a.lk2 = lam_k2;
    a.lam_init = li;
    a.sl2 = log2e_over_sqrt(d);
    a.B = B, a.T = T, a.H = H;
    a.softmax1 = softmax1;
    if (attn1) {
      a.attn = tout(*attn1);
      a.attn2 = tout(*attn2);
      a.lse = lse;
    }
    return launch_status(da::launch_prefill_v1_bf16(d, a, s));
  }
  da::V1F32Args a{};
  a.q1 = tin(q1), a.q2 = tin(q2), a.k1 = tin(k1), a.k2 = tin(k2), a.v = tin(v);
  a.out = tout(out);
  a.lq1 = lam_q1, a.lk1 = lam_k1, a.lq2 = lam_q2, a.lk2 = lam_k2;
  a.lam_init = li;
  a.sl2 = log2e_over_sqrt(d);
  a.B = B, a.H = H, a.T = T;
  a.softmax1 = softmax1;
  return launch_status(da::launch_v1_fp32(d, a, s));
}

static da_status v2_fwd_impl(int softmax1, int dtype, int B, int T, int Hq, int Hkv, int d, da_in q, da_in k,
                             da_in v,
                          da_in lam, da_out out, void* stream, const da_out* attn = nullptr,
                          float* lse = nullptr, const RopeK* rope = nullptr) {
  if (dtype != DA_FP32 && dtype != DA_BF16) return DA_E_DTYPE;
  if (B < 1 || T < 1 || Hq < 1 || Hkv < 1 || d < 1) return DA_E_SHAPE;
  if (rope && (!rope_theta_ok(rope->theta) || (long long)T >= kMaxRopePos)) return DA_E_SHAPE;
  if (Hq % Hkv != 0 || (Hq / Hkv) % 2 != 0) return DA_E_SHAPE;
  const int64_t mult = dtype == DA_BF16 ? 8 : 4;
  DA_TRY(check_in(q, mult));
  DA_TRY(check_in(k, mult));
  DA_TRY(check_in(v, mult));
  DA_TRY(check_logits(lam));
  DA_TRY(check_out(out, mult));
  DA_TRY(validate_v2_common(dtype, B, T, Hq, Hkv, d));
  if (k.st >= kMaxTokenStride || v.st >= kMaxTokenStride) return DA_E_UNSUPPORTED;
  if (!grid_fits((long long)B * (Hq / 2) * ((T + 31) / 32))) return DA_E_SHAPE;
  if (attn) {  // training forward
    DA_TRY(check_out(*attn, 8));
    if (!lse) return DA_E_NULL;
    if (!aligned(lse, 4)) return DA_E_LAYOUT;
  }
  if (rope && (!rope->ws || !aligned(rope->ws, 256) || rope->ws_bytes < rope_k_bytes(B, T, Hkv, d)))
    return DA_E_WORKSPACE;

  if (rope) {  // k rotated into the workspace as [B,T,Hkv,d]; q in the kernel's prologue
    da::RopeArgs r{};
    r.x = tin(k);
    r.out = TOut{rope->ws, (int64_t)T * Hkv * d, (int64_t)d, (int64_t)Hkv * d};
    r.B = B, r.T = T, r.H = Hkv, r.d = d, r.pos0 = 0;
    rope_tab(rope->theta, d, &r.w);
    const da_status st = launch_status(da::launch_rope_bf16(r, (hipStream_t)stream));
    if (st != DA_OK) return st;
    k = da_in{rope->ws, (int64_t)T * Hkv * d, (int64_t)d, (int64_t)Hkv * d};
  }
  da::PrefillArgs a{};
  a.q1 = a.q2 = tin(q);
  a.k1 = a.k2 = tin(k);
  a.v = tin(v);
  a.lam = tin(lam);
  a.out = tout(out);
  a.sl2 = log2e_over_sqrt(d);
  a.B = B, a.T = T, a.H = Hkv, a.G = Hq / Hkv;
  a.softmax1 = softmax1;
  if (attn) {
    a.attn = tout(*attn);
    a.lse = lse;
  }
  if (rope) {
    a.rope = 1;
    rope_tab(rope->theta, d, &a.rope_w);
  }
  return launch_status(da::launch_prefill_v2_bf16(d, a, (hipStream_t)stream));
}

// DIFF V2 backward: sizes of the two workspace regions.
struct BwdWs {
  size_t rows;  // bytes of each [B][Hq][Tp] fp32 array
  size_t total() const { return 2 * rows; }
};
static BwdWs bwd_ws(int B, int T, int Hq, int d) {
  (void)d;
  BwdWs w;
  w.rows = ((size_t)B * Hq * da::backward_padded_rows(T) * 4 + 255) / 256 * 256;
  return w;
}

static da_status v2_bwd_impl(int dtype, int B, int T, int Hq, int Hkv, int d, da_in q, da_in k, da_in v,
                             da_in lam, da_in attn, const float* lse, da_in dout, da_out dq, da_out dk, da_out dv,
                             da_out dlam, void* workspace, size_t workspace_bytes, void* stream) {
  if (dtype != DA_FP32 && dtype != DA_BF16) return DA_E_DTYPE;
  if (B < 1 || T < 1 || Hq < 1 || Hkv < 1 || d < 1) return DA_E_SHAPE;
  if (Hq % Hkv != 0 || (Hq / Hkv) % 2 != 0) return DA_E_SHAPE;
  for (const da_in* t : {&q, &k, &v, &attn, &dout}) DA_TRY(check_in(*t, 8));
  for (const da_out* t : {&dq, &dk, &dv}) DA_TRY(check_out(*t, 8));
  DA_TRY(check_logits(lam));
  da_in dl{dlam.ptr, dlam.sb, dlam.sh, dlam.st};
  DA_TRY(check_logits(dl));
  if (!lse) return DA_E_NULL;
  if (!aligned(lse, 4)) return DA_E_LAYOUT;
  DA_TRY(validate_v2_common(dtype, B, T, Hq, Hkv, d));
  if (q.st >= kMaxTokenStride || k.st >= kMaxTokenStride || v.st >= kMaxTokenStride ||
      dout.st >= kMaxTokenStride)
    return DA_E_UNSUPPORTED;
  const BwdWs w = bwd_ws(B, T, Hq, d);
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < w.total()) return DA_E_WORKSPACE;
  const int qt = (T + 127) / 128;
  if (!grid_fits((long long)B * Hq * qt) || !grid_fits(((long long)B * da::backward_padded_rows(T) * (Hq / 2) + 15) / 16))
    return DA_E_SHAPE;

  da::BwdArgs a{};
  a.q = tin(q), a.k = tin(k), a.v = tin(v), a.lam = tin(lam), a.attn = tin(attn), a.dout = tin(dout);
  a.lse = lse;
  a.dq = tout(dq), a.dk = tout(dk), a.dv = tout(dv), a.dlam = tout(dlam);
  a.Dw = (float*)workspace;
  a.lsew = (float*)((char*)workspace + w.rows);
  a.sl2 = log2e_over_sqrt(d);
  a.scale = (float)(1.0 / sqrt((double)d));
  a.B = B, a.T = T, a.Hq = Hq, a.Hkv = Hkv, a.G = Hq / Hkv;
  a.Tp = da::backward_padded_rows(T);
  return launch_status(da::launch_backward_v2_bf16(d, a, (hipStream_t)stream));
}

// DIFF V1 backward: workspace regions (each 256-byte aligned).
struct V1BwdWs {
  size_t dA, rows, lam;  // bytes of dD; of one [B][H][Tp] fp32 array; of the row terms of d lambda
  size_t total() const { return dA + 4 * rows + lam; }
};
static V1BwdWs v1_bwd_ws(int B, int H, int T, int d) {
  V1BwdWs w;
  w.dA = ((size_t)B * T * H * 2 * d * 2 + 255) / 256 * 256;
  w.rows = ((size_t)B * H * da::backward_padded_rows(T) * 4 + 255) / 256 * 256;
  w.lam = ((size_t)B * T * H * 4 + 255) / 256 * 256;
  return w;
}

static da_status v1_bwd_impl(int dtype, int B, int H, int T, int d, da_in q1, da_in q2, da_in k1, da_in k2,
                             da_in v, const float* lam_q1, const float* lam_k1, const float* lam_q2,
                             const float* lam_k2, int layer_index, da_in attn1, da_in attn2, const float* lse,
                             da_in dout, da_out dq1, da_out dq2, da_out dk1, da_out dk2, da_out dv, float* dlam_q1,
                             float* dlam_k1, float* dlam_q2, float* dlam_k2, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if (dtype != DA_FP32 && dtype != DA_BF16) return DA_E_DTYPE;
  if (B < 1 || H < 1 || T < 1 || d < 1 || layer_index < 0) return DA_E_SHAPE;
  for (const da_in* t : {&q1, &q2, &k1, &k2, &v, &attn1, &attn2, &dout}) DA_TRY(check_in(*t, 8));
  for (const da_out* t : {&dq1, &dq2, &dk1, &dk2, &dv}) DA_TRY(check_out(*t, 8));
  for (const float* p : {lam_q1, lam_k1, lam_q2, lam_k2, lse, (const float*)dlam_q1, (const float*)dlam_k1,
                         (const float*)dlam_q2, (const float*)dlam_k2}) {
    if (!p) return DA_E_NULL;
    if (!aligned(p, 4)) return DA_E_LAYOUT;
  }
  if (dtype != DA_BF16) return DA_E_UNSUPPORTED;
  if (d != 64 && d != 128) return DA_E_UNSUPPORTED;
  for (int64_t st : {q1.st, q2.st, k1.st, k2.st, v.st, (int64_t)H * 2 * d})
    if (st >= kMaxTokenStride) return DA_E_UNSUPPORTED;
  const V1BwdWs w = v1_bwd_ws(B, H, T, d);
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < w.total()) return DA_E_WORKSPACE;
  const int qt = (T + 127) / 128;
  if (!grid_fits(1 + 6LL * B * H * qt) || !grid_fits(((long long)B * da::backward_padded_rows(T) * H + 15) / 16))
    return DA_E_SHAPE;

  da::V1BwdArgs a{};
  a.q[0] = tin(q1), a.q[1] = tin(q2), a.k[0] = tin(k1), a.k[1] = tin(k2), a.v = tin(v);
  a.a[0] = tin(attn1), a.a[1] = tin(attn2), a.dout = tin(dout);
  a.lse = lse;
  a.lq1 = lam_q1, a.lk1 = lam_k1, a.lq2 = lam_q2, a.lk2 = lam_k2;
  a.dq[0] = tout(dq1), a.dq[1] = tout(dq2), a.dk[0] = tout(dk1), a.dk[1] = tout(dk2), a.dv = tout(dv);
  a.dlq1 = dlam_q1, a.dlk1 = dlam_k1, a.dlq2 = dlam_q2, a.dlk2 = dlam_k2;
  char* p = (char*)workspace;
  a.dD = (uint16_t*)p;
  p += w.dA;
  for (int m = 0; m < 2; ++m) {
    a.Dw[m] = (float*)(p + (2 * m) * w.rows);
    a.lsew[m] = (float*)(p + (2 * m + 1) * w.rows);
  }
  a.lamrow = (float*)(p + 4 * w.rows);
  a.lam_init = (float)diffattn_lambda_init(layer_index);
  a.sl2 = log2e_over_sqrt(d);
  a.scale = (float)(1.0 / sqrt((double)d));
  a.B = B, a.T = T, a.H = H;
  a.Tp = da::backward_padded_rows(T);
  return launch_status(da::launch_backward_v1_bf16(d, a, (hipStream_t)stream));
}

size_t diffattn_v2_decode_workspace_bytes(int B, int L, int Hq, int Hkv, int d) {
  return decode_ws_bytes(B, L, 1, Hq, Hkv, d, da::kDenseMaxChunk);
}

size_t diffattn_v2_decode_multi_workspace_bytes(int B, int L, int nq, int Hq, int Hkv, int d) {
  return decode_ws_bytes(B, L, nq, Hq, Hkv, d, da::kDenseMaxChunk);
}

size_t diffattn_v2_decode_paged_workspace_bytes(int B, int max_len, int nq, int Hq, int Hkv, int d) {
  return decode_ws_bytes(B, max_len, nq, Hq, Hkv, d, da::kPagedMaxChunk);
}

da_status diffattn_v1_fwd(int dtype, int B, int H, int T, int d, da_in q1, da_in q2, da_in k1, da_in k2,
                          da_in v, const float* lam_q1, const float* lam_k1, const float* lam_q2,
                          const float* lam_k2, int layer_index, da_out out, void* stream) {
  return v1_fwd_impl(0, dtype, B, H, T, d, q1, q2, k1, k2, v, lam_q1, lam_k1, lam_q2, lam_k2, layer_index, out,
                     stream);
}

da_status diffattn_v1_fwd_softmax1(int dtype, int B, int H, int T, int d, da_in q1, da_in q2, da_in k1,
                                   da_in k2, da_in v, const float* lam_q1, const float* lam_k1,
                                   const float* lam_q2, const float* lam_k2, int layer_index, da_out out,
                                   void* stream) {
  return v1_fwd_impl(1, dtype, B, H, T, d, q1, q2, k1, k2, v, lam_q1, lam_k1, lam_q2, lam_k2, layer_index, out,
                     stream);
}

da_status diffattn_v2_fwd(int dtype, int B, int T, int Hq, int Hkv, int d, da_in q, da_in k, da_in v,
                          da_in lam, da_out out, void* stream) {
  return v2_fwd_impl(0, dtype, B, T, Hq, Hkv, d, q, k, v, lam, out, stream);
}

da_status diffattn_v2_fwd_softmax1(int dtype, int B, int T, int Hq, int Hkv, int d, da_in q, da_in k,
                                   da_in v, da_in lam, da_out out, void* stream) {
  return v2_fwd_impl(1, dtype, B, T, Hq, Hkv, d, q, k, v, lam, out, stream);
}

da_status diffattn_v2_decode(int dtype, int B, int L, int Hq, int Hkv, int d, da_in q, da_in k_cache,
                             da_in v_cache, da_in lam, da_out out, void* workspace, size_t workspace_bytes,
                             void* stream) {
  return decode_impl(0, dtype, B, L, 1, Hq, Hkv, d, q, k_cache, v_cache, nullptr, lam, out, workspace,
                     workspace_bytes, stream);
}

da_status diffattn_v2_decode_noalloc(int dtype, int B, int L, int Hq, int Hkv, int d, da_in q, da_in k_cache,
                                     da_in v_cache, da_in lam, da_out out, void* stream) {
  if (!decode_sizes_ok(B, L, 1, Hq, Hkv, d)) return DA_E_SHAPE;
  // as many splits as the static scratch holds (at least one), never more
  // than the workspace entry point would use
  const size_t per_split = decode_split_bytes(B, 1, Hq, Hkv, d);
  if (per_split > kScratchBytes) return DA_E_SCRATCH;
  const size_t fit = kScratchBytes / per_split;
  const int max_splits = fit > 0x7fffffff ? 0x7fffffff : (int)fit;
  return decode_impl(0, dtype, B, L, 1, Hq, Hkv, d, q, k_cache, v_cache, nullptr, lam, out, nullptr, 0, stream,
                     0.f, max_splits, /*use_scratch=*/true);
}

size_t diffattn_v2_decode_noalloc_max_bytes(void) { return kScratchBytes; }

da_status diffattn_v2_decode_softmax1(int dtype, int B, int L, int Hq, int Hkv, int d, da_in q,
                                      da_in k_cache, da_in v_cache, da_in lam, da_out out, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  return decode_impl(1, dtype, B, L, 1, Hq, Hkv, d, q, k_cache, v_cache, nullptr, lam, out, workspace,
                     workspace_bytes, stream);
}

da_status diffattn_v2_decode_multi(int dtype, int B, int L, int nq, int Hq, int Hkv, int d, da_in q,
                                   da_in k_cache, da_in v_cache, da_in lam, da_out out, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  return decode_impl(0, dtype, B, L, nq, Hq, Hkv, d, q, k_cache, v_cache, nullptr, lam, out, workspace,
                     workspace_bytes, stream);
}

da_status diffattn_v2_decode_multi_softmax1(int dtype, int B, int L, int nq, int Hq, int Hkv, int d,
                                            da_in q, da_in k_cache, da_in v_cache, da_in lam, da_out out,
                                            void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(1, dtype, B, L, nq, Hq, Hkv, d, q, k_cache, v_cache, nullptr, lam, out, workspace,
                     workspace_bytes, stream);
}

da_status diffattn_v2_decode_paged(int dtype, int B, int max_len, int nq, int Hq, int Hkv, int d, da_in q,
                                   da_in k_pages, da_in v_pages, int num_pages, int page_size,
                                   const int32_t* block_table, int64_t bt_stride, const int32_t* seq_lens,
                                   da_in lam, da_out out, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  const PagedArgs pg{num_pages, page_size, block_table, bt_stride, seq_lens};
  return decode_impl(0, dtype, B, max_len, nq, Hq, Hkv, d, q, k_pages, v_pages, &pg, lam, out, workspace,
                     workspace_bytes, stream);
}

da_status diffattn_v2_decode_paged_softmax1(int dtype, int B, int max_len, int nq, int Hq, int Hkv, int d,
                                            da_in q, da_in k_pages, da_in v_pages, int num_pages, int page_size,
                                            const int32_t* block_table, int64_t bt_stride,
                                            const int32_t* seq_lens, da_in lam, da_out out, void* workspace,
                                            size_t workspace_bytes, void* stream) {
  const PagedArgs pg{num_pages, page_size, block_table, bt_stride, seq_lens};
  return decode_impl(1, dtype, B, max_len, nq, Hq, Hkv, d, q, k_pages, v_pages, &pg, lam, out, workspace,
                     workspace_bytes, stream);
}

da_status diffattn_v2_fwd_train(int dtype, int B, int T, int Hq, int Hkv, int d, da_in q, da_in k, da_in v,
                                da_in lam, da_out out, da_out attn, float* lse, void* stream) {
  return v2_fwd_impl(0, dtype, B, T, Hq, Hkv, d, q, k, v, lam, out, stream, &attn, lse);
}

da_status diffattn_v2_fwd_train_softmax1(int dtype, int B, int T, int Hq, int Hkv, int d, da_in q, da_in k,
                                         da_in v, da_in lam, da_out out, da_out attn, float* lse, void* stream) {
  return v2_fwd_impl(1, dtype, B, T, Hq, Hkv, d, q, k, v, lam, out, stream, &attn, lse);
}

size_t diffattn_v2_bwd_workspace_bytes(int B, int T, int Hq, int Hkv, int d) {
  if (B < 1 || T < 1 || Hq < 1 || Hkv < 1 || d < 1) return 0;
  if (Hq % Hkv != 0 || (Hq / Hkv) % 2 != 0) return 0;
  const BwdWs w = bwd_ws(B, T, Hq, d);
  return w.total();
}

da_status diffattn_v2_bwd(int dtype, int B, int T, int Hq, int Hkv, int d, da_in q, da_in k, da_in v,
                          da_in lam, da_in attn, const float* lse, da_in dout, da_out dq, da_out dk, da_out dv,
                          da_out dlam, void* workspace, size_t workspace_bytes, void* stream) {
  return v2_bwd_impl(dtype, B, T, Hq, Hkv, d, q, k, v, lam, attn, lse, dout, dq, dk, dv, dlam, workspace,
                     workspace_bytes, stream);
}

da_status diffattn_v1_fwd_train(int dtype, int B, int H, int T, int d, da_in q1, da_in q2, da_in k1, da_in k2,
                                da_in v, const float* lam_q1, const float* lam_k1, const float* lam_q2,
                                const float* lam_k2, int layer_index, da_out out, da_out attn1, da_out attn2,
                                float* lse, void* stream) {
  return v1_fwd_impl(0, dtype, B, H, T, d, q1, q2, k1, k2, v, lam_q1, lam_k1, lam_q2, lam_k2, layer_index, out,
                     stream, &attn1, &attn2, lse);
}

da_status diffattn_v1_fwd_train_softmax1(int dtype, int B, int H, int T, int d, da_in q1, da_in q2,
                                         da_in k1, da_in k2, da_in v, const float* lam_q1, const float* lam_k1,
                                         const float* lam_q2, const float* lam_k2, int layer_index, da_out out,
                                         da_out attn1, da_out attn2, float* lse, void* stream) {
  return v1_fwd_impl(1, dtype, B, H, T, d, q1, q2, k1, k2, v, lam_q1, lam_k1, lam_q2, lam_k2, layer_index, out,
                     stream, &attn1, &attn2, lse);
}

size_t diffattn_v1_bwd_workspace_bytes(int B, int H, int T, int d) {
  if (B < 1 || H < 1 || T < 1 || d < 1) return 0;
  return v1_bwd_ws(B, H, T, d).total();
}

da_status diffattn_v1_bwd(int dtype, int B, int H, int T, int d, da_in q1, da_in q2, da_in k1, da_in k2,
                          da_in v, const float* lam_q1, const float* lam_k1, const float* lam_q2,
                          const float* lam_k2, int layer_index, da_in attn1, da_in attn2, const float* lse,
                          da_in dout, da_out dq1, da_out dq2, da_out dk1, da_out dk2, da_out dv, float* dlam_q1,
                          float* dlam_k1, float* dlam_q2, float* dlam_k2, void* workspace, size_t workspace_bytes,
                          void* stream) {
  return v1_bwd_impl(dtype, B, H, T, d, q1, q2, k1, k2, v, lam_q1, lam_k1, lam_q2, lam_k2, layer_index, attn1,
                     attn2, lse, dout, dq1, dq2, dk1, dk2, dv, dlam_q1, dlam_k1, dlam_q2, dlam_k2, workspace,
                     workspace_bytes, stream);
}

size_t diffattn_v1_fwd_rope_workspace_bytes(int B, int H, int T, int d) {
  if (B < 1 || H < 1 || T < 1 || d < 1) return 0;
  return 2 * rope_k_bytes(B, T, H, d);
}

da_status diffattn_v1_fwd_rope(int dtype, int B, int H, int T, int d, da_in q1, da_in q2, da_in k1, da_in k2,
                               da_in v, const float* lam_q1, const float* lam_k1, const float* lam_q2,
                               const float* lam_k2, int layer_index, float theta, da_out out, void* workspace,
                               size_t workspace_bytes, void* stream) {
  const RopeK r{theta, workspace, workspace_bytes};
  return v1_fwd_impl(0, dtype, B, H, T, d, q1, q2, k1, k2, v, lam_q1, lam_k1, lam_q2, lam_k2, layer_index, out,
                     stream, nullptr, nullptr, nullptr, &r);
}

size_t diffattn_v2_fwd_rope_workspace_bytes(int B, int T, int Hkv, int d) {
  if (B < 1 || T < 1 || Hkv < 1 || d < 1) return 0;
  return rope_k_bytes(B, T, Hkv, d);
}

da_status diffattn_v2_fwd_rope(int dtype, int B, int T, int Hq, int Hkv, int d, da_in q, da_in k, da_in v,
                               da_in lam, float theta, da_out out, void* workspace, size_t workspace_bytes,
                               void* stream) {
  const RopeK r{theta, workspace, workspace_bytes};
  return v2_fwd_impl(0, dtype, B, T, Hq, Hkv, d, q, k, v, lam, out, stream, nullptr, nullptr, &r);
}

da_status diffattn_v2_decode_rope(int dtype, int B, int L, int Hq, int Hkv, int d, da_in q, da_in k_cache,
                                  da_in v_cache, da_in lam, float theta, da_out out, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  if (!rope_theta_ok(theta)) return DA_E_SHAPE;
  return decode_impl(0, dtype, B, L, 1, Hq, Hkv, d, q, k_cache, v_cache, nullptr, lam, out, workspace,
                     workspace_bytes, stream, theta);
}

da_status diffattn_v2_decode_paged_rope(int dtype, int B, int max_len, int nq, int Hq, int Hkv, int d, da_in q,
                                        da_in k_pages, da_in v_pages, int num_pages, int page_size,
                                        const int32_t* block_table, int64_t bt_stride, const int32_t* seq_lens,
                                        da_in lam, float theta, da_out out, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  if (!rope_theta_ok(theta)) return DA_E_SHAPE;
  const PagedArgs pg{num_pages, page_size, block_table, bt_stride, seq_lens};
  return decode_impl(0, dtype, B, max_len, nq, Hq, Hkv, d, q, k_pages, v_pages, &pg, lam, out, workspace,
                     workspace_bytes, stream, theta);
}

da_status diffattn_v1_fwd_softmax1_rope(int dtype, int B, int H, int T, int d, da_in q1, da_in q2, da_in k1,
                                       da_in k2, da_in v, const float* lam_q1, const float* lam_k1,
                                       const float* lam_q2, const float* lam_k2, int layer_index, float theta,
                                       da_out out, void* workspace, size_t workspace_bytes, void* stream) {
  const RopeK r{theta, workspace, workspace_bytes};
  return v1_fwd_impl(1, dtype, B, H, T, d, q1, q2, k1, k2, v, lam_q1, lam_k1, lam_q2, lam_k2, layer_index, out,
                     stream, nullptr, nullptr, nullptr, &r);
}

da_status diffattn_v2_fwd_softmax1_rope(int dtype, int B, int T, int Hq, int Hkv, int d, da_in q, da_in k,
                                       da_in v, da_in lam, float theta, da_out out, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  const RopeK r{theta, workspace, workspace_bytes};
  return v2_fwd_impl(1, dtype, B, T, Hq, Hkv, d, q, k, v, lam, out, stream, nullptr, nullptr, &r);
}

da_status diffattn_v2_decode_softmax1_rope(int dtype, int B, int L, int Hq, int Hkv, int d, da_in q,
                                          da_in k_cache, da_in v_cache, da_in lam, float theta, da_out out,
                                          void* workspace, size_t workspace_bytes, void* stream) {
  if (!rope_theta_ok(theta)) return DA_E_SHAPE;
  return decode_impl(1, dtype, B, L, 1, Hq, Hkv, d, q, k_cache, v_cache, nullptr, lam, out, workspace,
                     workspace_bytes, stream, theta);
}

da_status diffattn_v2_decode_paged_softmax1_rope(int dtype, int B, int max_len, int nq, int Hq, int Hkv, int d,
                                                da_in q, da_in k_pages, da_in v_pages, int num_pages, int page_size,
                                                const int32_t* block_table, int64_t bt_stride,
                                                const int32_t* seq_lens, da_in lam, float theta, da_out out,
                                                void* workspace, size_t workspace_bytes, void* stream) {
  if (!rope_theta_ok(theta)) return DA_E_SHAPE;
  const PagedArgs pg{num_pages, page_size, block_table, bt_stride, seq_lens};
  return decode_impl(1, dtype, B, max_len, nq, Hq, Hkv, d, q, k_pages, v_pages, &pg, lam, out, workspace,
                     workspace_bytes, stream, theta);
}

da_status diffattn_rope(int dtype, int B, int T, int H, int d, da_in x, da_out out, float theta, int pos0,
                        void* stream) {
  if (dtype != DA_FP32 && dtype != DA_BF16) return DA_E_DTYPE;
  if (B < 1 || T < 1 || H < 1 || d < 1 || pos0 < 0) return DA_E_SHAPE;
  if (!rope_theta_ok(theta) || (long long)pos0 + T >= kMaxRopePos) return DA_E_SHAPE;
  DA_TRY(check_in(x, 8));
  DA_TRY(check_out(out, 8));
  if (dtype != DA_BF16) return DA_E_UNSUPPORTED;
  if (d % 8 != 0 || d > 256) return DA_E_UNSUPPORTED;
  if (!grid_fits(((long long)B * T * H * (d / 4) + 255) / 256)) return DA_E_SHAPE;
  da::RopeArgs r{};
  r.x = tin(x);
  r.out = tout(out);
  r.B = B, r.T = T, r.H = H, r.d = d, r.pos0 = pos0;
  rope_tab(theta, d, &r.w);
  return launch_status(da::launch_rope_bf16(r, (hipStream_t)stream));
}

da_status diffattn_v2_lambda_proj(int dtype, int B, int T, int dm, int P, da_in x, da_in w, da_in out,
                                  void* stream) {
  if (dtype != DA_FP32 && dtype != DA_BF16) return DA_E_DTYPE;
  if (B < 1 || T < 1 || dm < 1 || P < 1) return DA_E_SHAPE;
  DA_TRY(check_in(x, 8));
  DA_TRY(check_in(w, 8));
  DA_TRY(check_logits(out));
  if (dtype != DA_BF16) return DA_E_UNSUPPORTED;
  if (dm % 128 != 0) return DA_E_UNSUPPORTED;
  if (!grid_fits(((long long)B * T + 31) / 32 * ((P + 31) / 32))) return DA_E_SHAPE;
  da::LamProjArgs a{};
  a.x = tin(x);
  a.w = tin(w);
  a.out = TOut{(void*)out.ptr, out.sb, out.sh, out.st};
  a.B = B, a.T = T, a.dm = dm, a.P = P;
  return launch_status(da::launch_lambda_proj_bf16(a, (hipStream_t)stream));
}

}  // extern "C"

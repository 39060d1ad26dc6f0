// Drives the C ABI's host code (gdn_api.cpp, linked with api_stubs.cpp: no
// GPU, no HIP runtime) under AddressSanitizer and UndefinedBehaviorSanitizer:
// every validation error of the prefill, decode, output-gate and
// cu_seqlens entry points, the workspace layouts, calls that pass
// validation (ending in GDN_ERR_HIP at the stubbed launch), the
// no-allocation entry point and the graph cache's bookkeeping.  Descriptors
// carry fake device addresses that are never dereferenced.  Exit status 0
// means every status matched; a sanitizer report aborts the run.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <initializer_list>

#include "gdn.h"

namespace {

int fails = 0;

void expect(int got, int want, const char* what) {
  if (got != want) {
    std::printf("FAIL %s: got %d want %d (%s)\n", what, got, want, gdn_last_error());
    ++fails;
  }
}

gdn_tensor tensor(std::initializer_list<int64_t> shape, int dtype, uintptr_t addr = 0x100000) {
  gdn_tensor t;
  std::memset(&t, 0, sizeof t);
  t.data = (void*)addr;
  t.dtype = dtype;
  t.ndim = (int32_t)shape.size();
  int i = 0;
  for (int64_t s : shape) t.shape[i++] = s;
  int64_t acc = 1;
  for (int j = t.ndim - 1; j >= 0; --j) {
    t.stride[j] = acc;
    acc *= t.shape[j];
  }
  return t;
}

struct Args {
  gdn_tensor q, k, v, g, b, out;
};

Args base(int64_t T = 128, int64_t hk = 2, int64_t hv = 4, int64_t dk = 64, int64_t dv = 64,
          int dt = GDN_DTYPE_BF16) {
  return Args{tensor({T, hk, dk}, dt), tensor({T, hk, dk}, dt), tensor({T, hv, dv}, dt),
              tensor({T, hv}, GDN_DTYPE_F32), tensor({T, hv}, GDN_DTYPE_F32), tensor({T, hv, dv}, dt)};
}

int prefill(Args& a, const gdn_tensor* cu = nullptr, const gdn_options* o = nullptr,
            const gdn_tensor* init = nullptr, gdn_tensor* fin = nullptr, size_t ws_bytes = (size_t)1 << 40,
            uintptr_t ws = 0x1000000) {
  return gdn_prefill_ex(&a.q, &a.k, &a.v, &a.g, &a.b, cu, init, &a.out, fin, o, (void*)ws, ws_bytes,
                        nullptr);
}

}  // namespace

int main() {
  expect(gdn_abi_version(), GDN_ABI_VERSION, "abi version");
  for (int s = -9; s <= 1; ++s) (void)gdn_status_string(s);

  // the prefill's validation errors
  {
    Args a = base();
    expect(gdn_prefill_ex(nullptr, &a.k, &a.v, &a.g, &a.b, nullptr, nullptr, &a.out, nullptr,
                          nullptr, (void*)0x1000000, 1 << 30, nullptr), GDN_ERR_NULL_ARG, "null q");
    Args d = base(); d.k = tensor({128, 2, 64}, GDN_DTYPE_F32);
    expect(prefill(d), GDN_ERR_DTYPE, "dtype k");
    Args s = base(); s.v = tensor({127, 4, 64}, GDN_DTYPE_BF16);
    expect(prefill(s), GDN_ERR_SHAPE, "v tokens");
    Args h = base(); h.q = h.k = tensor({128, 2, 96}, GDN_DTYPE_BF16);
    expect(prefill(h), GDN_ERR_UNSUPPORTED, "head dim 96");
    Args m = base(); m.q = tensor({128, 2, 64}, GDN_DTYPE_BF16, 0x100002);
    expect(prefill(m), GDN_ERR_LAYOUT, "misaligned q");
    Args l = base(); l.v.stride[2] = 2;
    expect(prefill(l), GDN_ERR_LAYOUT, "last stride");
    Args w = base();
    expect(prefill(w, nullptr, nullptr, nullptr, nullptr, 10), GDN_ERR_WORKSPACE, "small workspace");
    expect(prefill(w, nullptr, nullptr, nullptr, nullptr, (size_t)1 << 40, 0x1000010), GDN_ERR_WORKSPACE,
           "misaligned workspace");
    gdn_options o;
    gdn_default_options(&o);
    o.chunk = 48;
    expect(prefill(w, nullptr, &o), GDN_ERR_UNSUPPORTED, "chunk 48");
    gdn_default_options(&o);
    o.flags = 32;
    expect(prefill(w, nullptr, &o), GDN_ERR_SHAPE, "unknown flag");
    gdn_default_options(&o);
    o.flags = GDN_FLAG_QKV_CONV;
    expect(prefill(w, nullptr, &o), GDN_ERR_NULL_ARG, "convolution without taps");
    o.conv_weight = (const float*)0x200000;
    o.conv_width = 5;
    expect(prefill(w, nullptr, &o), GDN_ERR_SHAPE, "convolution width 5");
    o.conv_width = 3;
    o.conv_state_in = (const void*)0x200008;
    expect(prefill(w, nullptr, &o), GDN_ERR_LAYOUT, "misaligned convolution history");
    gdn_default_options(&o);
    o.flags = GDN_FLAG_OUTPUT_GATE;
    expect(prefill(w, nullptr, &o), GDN_ERR_NULL_ARG, "gate without z");
    o.gate_z = (const void*)0x200008;
    expect(prefill(w, nullptr, &o), GDN_ERR_LAYOUT, "misaligned z");
    gdn_default_options(&o);
    o.norm_eps = -1.f;
    expect(prefill(w, nullptr, &o), GDN_ERR_SHAPE, "negative norm eps");
    gdn_tensor st_bad = tensor({2, 4, 64, 64}, GDN_DTYPE_F32);
    gdn_tensor cu = tensor({4}, GDN_DTYPE_I32);
    expect(prefill(w, &cu, nullptr, &st_bad), GDN_ERR_SHAPE, "init shape");
  }
  // calls that pass validation end at the stubbed launches
  {
    Args a = base();
    expect(prefill(a), GDN_ERR_HIP, "valid one sequence");
    gdn_tensor cu = tensor({4}, GDN_DTYPE_I32);
    gdn_tensor st = tensor({3, 4, 64, 64}, GDN_DTYPE_F32);
    expect(prefill(a, &cu, nullptr, &st, &st), GDN_ERR_HIP, "valid packed");
    gdn_options o;
    gdn_default_options(&o);
    o.flags = GDN_FLAG_DECAY_PROJ | GDN_FLAG_OUTPUT_GATE | GDN_FLAG_BETA_LOGITS;
    o.gate_z = (const void*)0x200000;
    expect(prefill(a, nullptr, &o), GDN_ERR_HIP, "valid gated");
    setenv("GDN_DEBUG_CHECK", "1", 1);
    expect(prefill(a, &cu), GDN_ERR_HIP, "debug check (no device)");
    unsetenv("GDN_DEBUG_CHECK");
    expect(gdn_prefill_noalloc(&a.q, &a.k, &a.v, &a.g, &a.b, nullptr, nullptr, &a.out, nullptr, nullptr,
                               nullptr), GDN_ERR_HIP, "noalloc");
    Args big = base(1 << 20, 16, 16, 128, 128);
    expect(gdn_prefill_noalloc(&big.q, &big.k, &big.v, &big.g, &big.b, nullptr, nullptr, &big.out,
                               nullptr, nullptr, nullptr), GDN_ERR_WORKSPACE, "noalloc oversize");
  }
  // workspace layouts, one-pass and two-level
  {
    Args a = base(4096, 16, 16, 128, 128);
    size_t n = 0;
    expect(gdn_workspace_size(&a.q, &a.k, &a.v, nullptr, nullptr, &n), GDN_OK, "workspace size");
    gdn_workspace_layout lay;
    gdn_options o;
    gdn_default_options(&o);
    o.scan_split = GDN_SCAN_TWO_LEVEL;
    expect(gdn_get_workspace_layout(&a.q, &a.k, &a.v, nullptr, &o, &lay), GDN_OK, "two-level layout");
    if (lay.split_chunks != 34 || lay.total_bytes <= n) {
      std::printf("FAIL two-level layout values\n");
      ++fails;
    }
    gdn_tensor cu = tensor({256}, GDN_DTYPE_I32);
    expect(gdn_get_workspace_layout(&a.q, &a.k, &a.v, &cu, nullptr, &lay), GDN_OK, "packed layout");
    expect(gdn_get_workspace_layout(&a.q, &a.k, &a.v, &cu, &o, &lay), GDN_ERR_UNSUPPORTED, "packed two-level");
  }
  // decode
  {
    gdn_tensor q = tensor({3, 1, 16}, GDN_DTYPE_BF16), v = tensor({3, 2, 16}, GDN_DTYPE_BF16);
    gdn_tensor g = tensor({3, 2}, GDN_DTYPE_F32), st = tensor({3, 2, 16, 16}, GDN_DTYPE_F32);
    expect(gdn_decode(&q, &q, &v, &g, &g, &st, &v, nullptr, nullptr), GDN_ERR_HIP, "decode valid");
    gdn_tensor st_bad = tensor({3, 2, 16, 8}, GDN_DTYPE_F32);
    expect(gdn_decode(&q, &q, &v, &g, &g, &st_bad, &v, nullptr, nullptr), GDN_ERR_SHAPE, "decode state");
    gdn_options o;
    gdn_default_options(&o);
    o.flags = GDN_FLAG_OUTPUT_GATE;
    expect(gdn_decode(&q, &q, &v, &g, &g, &st, &v, &o, nullptr), GDN_ERR_NULL_ARG, "decode gate without z");
  }
  // the output gate
  {
    gdn_tensor x = tensor({10, 4, 64}, GDN_DTYPE_BF16);
    expect(gdn_output_gate(&x, &x, nullptr, 1e-6f, &x, nullptr), GDN_ERR_HIP, "gate valid");
    gdn_tensor y = tensor({10, 4, 48}, GDN_DTYPE_BF16);
    expect(gdn_output_gate(&y, &y, nullptr, 1e-6f, &y, nullptr), GDN_ERR_UNSUPPORTED, "gate dv 48");
    gdn_tensor e = tensor({0, 4, 64}, GDN_DTYPE_BF16);
    expect(gdn_output_gate(&e, &e, nullptr, 1e-6f, &e, nullptr), GDN_OK, "gate no rows");
    expect(gdn_output_gate(&x, nullptr, nullptr, 1e-6f, &x, nullptr), GDN_ERR_NULL_ARG, "gate null z");
  }
  // cu_seqlens
  {
    const int32_t good[] = {0, 3, 3, 7};
    const int32_t dec[] = {0, 5, 4, 9};
    const int32_t past[] = {0, 5, 10};
    expect(gdn_check_cu_seqlens(good, 3, 7), GDN_OK, "cu good");
    expect(gdn_check_cu_seqlens(dec, 3, 9), GDN_ERR_INPUT, "cu decreasing");
    expect(gdn_check_cu_seqlens(past, 2, 9), GDN_ERR_INPUT, "cu past end");
    expect(gdn_check_cu_seqlens(nullptr, 2, 9), GDN_ERR_NULL_ARG, "cu null");
  }
  // the graph cache's bookkeeping (capture itself needs a device)
  {
    gdn_graph_cache* c = nullptr;
    expect(gdn_graph_cache_create(0, &c), GDN_ERR_SHAPE, "cache capacity 0");
    expect(gdn_graph_cache_create(4, &c), GDN_OK, "cache create");
    Args a = base();
    Args bad = base(); bad.k = tensor({128, 2, 64}, GDN_DTYPE_F32);
    expect(gdn_prefill_graph(c, &bad.q, &bad.k, &bad.v, &bad.g, &bad.b, nullptr, nullptr, &bad.out, nullptr,
                             nullptr, (void*)0x1000000, (size_t)1 << 40, nullptr), GDN_ERR_DTYPE, "graph dtype");
    expect(gdn_prefill_graph(c, &a.q, &a.k, &a.v, &a.g, &a.b, nullptr, nullptr, &a.out, nullptr, nullptr,
                             (void*)0x1000000, (size_t)1 << 40, nullptr), GDN_ERR_HIP, "graph eager fallback");
    int entries = -1;
    int64_t hits = -1, misses = -1, updates = -1, fallbacks = -1;
    expect(gdn_graph_cache_stats(c, &entries, &hits, &misses, &updates, &fallbacks), GDN_OK, "cache stats");
    if (entries != 0 || misses != 1 || updates != 0 || fallbacks != 1) {
      std::printf("FAIL cache counts %d %lld %lld\n", entries, (long long)misses, (long long)fallbacks);
      ++fails;
    }
    gdn_graph_cache_clear(c);
    gdn_graph_cache_destroy(c);
  }
  std::printf("host code under sanitizers: %d failure(s)\n", fails);
  return fails ? 1 : 0;
}

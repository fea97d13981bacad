// Host-only driver of libgdn's C ABI for the AddressSanitizer /
// UndefinedBehaviorSanitizer build: every argument check, size query and
// error path of the boundary (include/gdn.h), with descriptors at and past
// the documented limits and pointer patterns that are null, misaligned or
// overlapping.  No call here reaches a kernel launch (every case fails its
// checks or only sizes), so it runs where there is no GPU.  Each result is
// compared with the status the header documents; any mismatch, or any
// sanitizer report, fails the run.
#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "gdn.h"

namespace {

int failures = 0;

void expect(const char* what, int got, int want) {
  if (got != want) {
    std::printf("FAIL %s: got %d want %d (%s)\n", what, got, want, gdn_last_error());
    ++failures;
  }
}

gdn_desc desc(int B, int H, int T, int S, int D, int io = GDN_BF16, int mode = GDN_BETA_ERASE, uint32_t flags = 0) {
  gdn_desc d;
  d.abi_version = GDN_ABI_VERSION;
  d.B = B; d.H = H; d.T = T; d.S = S; d.D = D;
  d.io_dtype = io; d.beta_mode = mode; d.flags = flags;
  return d;
}

// fake device addresses: never dereferenced by the host checks
char* at(uintptr_t x) { return reinterpret_cast<char*>(x); }

struct Bufs {
  const void *q, *k, *v;
  const float *g, *b, *sin;
  void* o;
  float *sout, *nrm;
  void* ws;
  size_t wsb;
};

// disjoint, aligned buffers for desc d (sizes from the shapes)
Bufs good(const gdn_desc& d, size_t wsb) {
  const size_t esz = d.io_dtype == GDN_F32 ? 4 : d.io_dtype == GDN_BF16 ? 2 : 1;
  const size_t big = (size_t)1 << 40;   // far apart
  Bufs b;
  b.q = at(big * 1); b.k = at(big * 2); b.v = at(big * 3);
  b.g = (const float*)at(big * 4); b.b = (const float*)at(big * 5); b.sin = (const float*)at(big * 6);
  b.o = at(big * 7); b.sout = (float*)at(big * 8); b.nrm = (float*)at(big * 9);
  b.ws = at(big * 10); b.wsb = wsb;
  (void)esz;
  return b;
}

gdn_status check(const gdn_desc& d, const Bufs& b, int step) {
  return gdn_check_args(&d, b.q, b.k, b.v, b.g, b.b, b.sin, b.o, b.sout, b.nrm, b.ws, b.wsb, step);
}

}  // namespace

int main() {
  expect("abi version", gdn_abi_version(), GDN_ABI_VERSION);
  for (int s = -3; s < 14; ++s) {
    const char* txt = gdn_status_string((gdn_status)s);
    if (!txt || !*txt) { std::printf("FAIL status string %d\n", s); ++failures; }
  }
  (void)gdn_last_error();

  // --- sizes over a grid of shapes, valid and not
  const int dims[] = {-1, 0, 1, 2, 7, 16, 81, 961, 1024, 1025, 4096, 65536, INT_MAX};
  const int ds[] = {0, 8, 16, 48, 112, 128, 144};
  const int ios[] = {-1, GDN_F32, GDN_BF16, GDN_FP8_E4M3, 3};
  size_t acc = 0;
  for (int B : {1, 2, 1 << 20, INT_MAX})
    for (int T : dims)
      for (int S : dims)
        for (int D : ds)
          for (int io : ios) {
            gdn_desc d = desc(B, 20, T, S, D, io);
            acc += gdn_workspace_size(&d) + gdn_workspace_min_size(&d) + gdn_backward_workspace_size(&d) +
                   gdn_saved_size(&d) + gdn_backward_saved_workspace_size(&d);
          }
  gdn_desc bad_abi = desc(1, 1, 1, 16, 16);
  bad_abi.abi_version = 99;
  expect("sizes of a bad abi", (int)(gdn_workspace_size(&bad_abi) + gdn_saved_size(&bad_abi)), 0);

  // --- the forward's argument checks
  const gdn_desc d = desc(1, 4, 9, 33, 64);
  const size_t wmin = gdn_workspace_min_size(&d);
  Bufs b = good(d, wmin + 4096);
  expect("valid", check(d, b, 0), GDN_OK);
  expect("valid step", check(d, b, 1), GDN_OK);
  { Bufs x = b; x.sin = nullptr; expect("step without state", check(d, x, 1), GDN_ERR_NULL); }
  { Bufs x = b; x.q = nullptr; expect("null q", check(d, x, 0), GDN_ERR_NULL); }
  { Bufs x = b; x.o = nullptr; expect("null o", check(d, x, 0), GDN_ERR_NULL); }
  { Bufs x = b; x.g = nullptr; expect("null gamma", check(d, x, 0), GDN_ERR_NULL); }
  { Bufs x = b; x.ws = nullptr; expect("null workspace", check(d, x, 0), GDN_ERR_WORKSPACE); }
  { Bufs x = b; x.wsb = 16; expect("short workspace", check(d, x, 0), GDN_ERR_WORKSPACE); }
  { Bufs x = b; x.q = at((uintptr_t)b.q + 2); expect("misaligned q", check(d, x, 0), GDN_ERR_ALIGN); }
  { Bufs x = b; x.o = at((uintptr_t)b.o + 8); expect("misaligned o", check(d, x, 0), GDN_ERR_ALIGN); }
  { Bufs x = b; x.g = (const float*)at((uintptr_t)b.g + 1); expect("misaligned gamma", check(d, x, 0), GDN_ERR_ALIGN); }
  { Bufs x = b; x.ws = at((uintptr_t)b.ws + 64); expect("misaligned workspace", check(d, x, 0), GDN_ERR_ALIGN); }
  { Bufs x = b; x.o = const_cast<void*>(b.q); expect("o aliases q", check(d, x, 0), GDN_ERR_ALIAS); }
  { Bufs x = b; x.o = at((uintptr_t)b.k + 4096); expect("o overlaps k", check(d, x, 0), GDN_ERR_ALIAS); }
  { Bufs x = b; x.sout = (float*)b.nrm; expect("state_out aliases norms", check(d, x, 0), GDN_ERR_ALIAS); }
  { Bufs x = b; x.ws = const_cast<void*>(b.v); expect("workspace aliases v", check(d, x, 0), GDN_ERR_ALIAS); }
  { Bufs x = b; x.sout = const_cast<float*>(b.sin); expect("in-place state", check(d, x, 1), GDN_OK); }
  expect("abi", check(bad_abi, good(bad_abi, 1 << 30), 0), GDN_ERR_ABI);
  for (int D : {8, 24, 144}) {
    gdn_desc e = desc(1, 1, 1, 16, D);
    expect("unsupported D", check(e, good(e, 1 << 30), 0), GDN_ERR_UNSUPPORTED);
  }
  for (int D : {0, -16}) {
    gdn_desc e = desc(1, 1, 1, 16, D);
    expect("D out of range", check(e, good(e, 1 << 30), 0), GDN_ERR_SHAPE);
  }
  for (int io : {-1, 3, 77}) {
    gdn_desc e = desc(1, 1, 1, 16, 16, io);
    expect("bad dtype", check(e, good(e, 1 << 30), 0), GDN_ERR_DTYPE);
  }
  {
    gdn_desc e = desc(1, 1, 1, 16, 16, GDN_BF16, 5);
    expect("bad beta mode", check(e, good(e, 1 << 30), 0), GDN_ERR_DTYPE);
  }
  for (int x : {0, -1}) {
    gdn_desc e = desc(x, 1, 1, 16, 16);
    expect("bad B", check(e, good(e, 1 << 30), 0), GDN_ERR_SHAPE);
    e = desc(1, 1, 1, x, 16);
    expect("bad S", check(e, good(e, 1 << 30), 0), GDN_ERR_SHAPE);
  }
  {
    gdn_desc e = desc(INT_MAX, INT_MAX, INT_MAX, INT_MAX, 128);
    expect("overflowing sizes", check(e, good(e, (size_t)-1), 0), GDN_ERR_SHAPE);
  }
  {
    gdn_desc e = desc(1, 1, 1, 16, 16, GDN_BF16, GDN_BETA_ERASE, 0x80u);
    expect("unknown flag", check(e, good(e, 1 << 30), 0), GDN_ERR_UNSUPPORTED);
    e.flags = GDN_FLAG_THREE_PASS | GDN_FLAG_ONE_LAUNCH;
    expect("exclusive flags", check(e, good(e, 1 << 30), 0), GDN_ERR_UNSUPPORTED);
    e = desc(1, 1, 1, 16, 16, GDN_FP8_E4M3, GDN_BETA_ERASE, GDN_FLAG_DIRECT);
    expect("direct with e4m3", check(e, good(e, 1 << 30), 0), GDN_ERR_UNSUPPORTED);
  }
  // entry points fail their checks before touching a device
  expect("forward null desc", gdn_frame_forward(nullptr, b.q, b.k, b.v, b.g, b.b, nullptr, b.o, nullptr, nullptr,
                                                b.ws, b.wsb, nullptr), GDN_ERR_NULL);
  expect("forward null q", gdn_frame_forward(&d, nullptr, b.k, b.v, b.g, b.b, nullptr, b.o, nullptr, nullptr,
                                             b.ws, b.wsb, nullptr), GDN_ERR_NULL);
  expect("step without state", gdn_frame_step(&d, b.q, b.k, b.v, b.g, b.b, nullptr, b.o, nullptr, nullptr,
                                               b.ws, b.wsb, nullptr), GDN_ERR_NULL);
  expect("noalloc null o", gdn_frame_forward_noalloc(&d, b.q, b.k, b.v, b.g, b.b, nullptr, nullptr, nullptr,
                                                     nullptr, nullptr), GDN_ERR_NULL);
  {
    gdn_desc e = d;
    e.flags = GDN_FLAG_TIME_KERNELS;
    expect("noalloc timed", gdn_frame_forward_noalloc(&e, b.q, b.k, b.v, b.g, b.b, nullptr, b.o, nullptr,
                                                      nullptr, nullptr), GDN_ERR_UNSUPPORTED);
  }

  // --- backward and the training pair
  const size_t bw = gdn_backward_workspace_size(&d), sv = gdn_saved_size(&d), bsw = gdn_backward_saved_workspace_size(&d);
  if (!bw || !sv || !bsw) { std::printf("FAIL backward sizes %zu %zu %zu\n", bw, sv, bsw); ++failures; }
  {
    gdn_desc e = desc(1, 1, 1025, 16, 16);
    expect("backward T > 1024", (int)gdn_backward_workspace_size(&e), 0);
    e = desc(1, 1, 4, 16, 16, GDN_FP8_E4M3);
    expect("backward e4m3", (int)gdn_saved_size(&e), 0);
  }
  expect("backward null d_out",
         gdn_frame_backward(&d, b.q, b.k, b.v, b.g, b.b, nullptr, nullptr, nullptr, at(1ull << 44), nullptr, nullptr,
                            nullptr, nullptr, nullptr, b.ws, bw, nullptr), GDN_ERR_NULL);
  expect("backward dq aliases q",
         gdn_frame_backward(&d, b.q, b.k, b.v, b.g, b.b, nullptr, at(1ull << 45), nullptr, const_cast<void*>(b.q),
                            nullptr, nullptr, nullptr, nullptr, nullptr, b.ws, bw, nullptr), GDN_ERR_ALIAS);
  expect("train short saved", gdn_frame_forward_train(&d, b.q, b.k, b.v, b.g, b.b, nullptr, b.o, nullptr, nullptr,
                                                      at(1ull << 46), 64, nullptr), GDN_ERR_WORKSPACE);
  expect("backward_saved misaligned saved",
         gdn_frame_backward_saved(&d, b.q, b.k, b.v, b.g, b.b, at((1ull << 46) + 16), sv, at(1ull << 45), nullptr,
                                  at(1ull << 47), nullptr, nullptr, nullptr, nullptr, nullptr, b.ws, bsw, nullptr),
         GDN_ERR_ALIGN);

  // --- temporal convolution
  gdn_tconv_desc t;
  t.abi_version = GDN_ABI_VERSION; t.B = 2; t.T = 13; t.S = 40; t.C = 64; t.chunk = 4; t.io_dtype = GDN_BF16; t.flags = 0;
  const float* w = (const float*)at(1ull << 41);
  const float* bias = (const float*)at(2ull << 41);
  expect("tconv valid", gdn_tconv_check_args(&t, b.q, w, bias, nullptr, b.o, nullptr), GDN_OK);
  expect("tconv null x", gdn_tconv_check_args(&t, nullptr, w, bias, nullptr, b.o, nullptr), GDN_ERR_NULL);
  expect("tconv y aliases x", gdn_tconv_check_args(&t, b.q, w, bias, nullptr, const_cast<void*>(b.q), nullptr),
         GDN_ERR_ALIAS);
  expect("tconv misaligned y", gdn_tconv_check_args(&t, b.q, w, bias, nullptr, at((uintptr_t)b.o + 2), nullptr),
         GDN_ERR_ALIGN);
  for (int c : {0, -1}) {
    gdn_tconv_desc u = t;
    u.chunk = c;
    expect("tconv bad chunk", gdn_tconv_check_args(&u, b.q, w, bias, nullptr, b.o, nullptr), GDN_ERR_SHAPE);
  }
  {
    gdn_tconv_desc u = t;
    u.B = INT_MAX; u.T = INT_MAX; u.S = INT_MAX; u.C = INT_MAX & ~7;
    expect("tconv overflow", gdn_tconv_check_args(&u, b.q, w, bias, nullptr, b.o, nullptr), GDN_ERR_SHAPE);
    u = t;
    u.io_dtype = GDN_FP8_E4M3;
    expect("tconv e4m3", gdn_tconv_check_args(&u, b.q, w, bias, nullptr, b.o, nullptr), GDN_ERR_DTYPE);
  }
  expect("tconv forward null desc", gdn_tconv_forward(nullptr, b.q, w, bias, nullptr, b.o, nullptr, nullptr),
         GDN_ERR_NULL);

  // --- block-causal attention
  gdn_attn_desc a;
  a.abi_version = GDN_ABI_VERSION; a.B = 1; a.H = 2; a.Tq = 4; a.Tk = 12; a.S = 40; a.D = 64; a.chunk = 4;
  a.io_dtype = GDN_BF16; a.flags = 0; a.scale = 0.f;
  expect("attn valid", gdn_attention_check_args(&a, b.q, b.k, b.v, b.o, nullptr, 0), GDN_OK);
  expect("attn null v", gdn_attention_check_args(&a, b.q, b.k, nullptr, b.o, nullptr, 0), GDN_ERR_NULL);
  expect("attn o aliases k", gdn_attention_check_args(&a, b.q, b.k, b.v, const_cast<void*>(b.k), nullptr, 0),
         GDN_ERR_ALIAS);
  {
    gdn_attn_desc e = a;
    e.Tq = 13;
    expect("attn Tq > Tk", gdn_attention_check_args(&e, b.q, b.k, b.v, b.o, nullptr, 0), GDN_ERR_SHAPE);
    e = a;
    e.scale = -1.f;
    expect("attn negative scale", gdn_attention_check_args(&e, b.q, b.k, b.v, b.o, nullptr, 0), GDN_ERR_SHAPE);
    e = a;
    e.D = 72;
    expect("attn bad D", gdn_attention_check_args(&e, b.q, b.k, b.v, b.o, nullptr, 0), GDN_ERR_UNSUPPORTED);
    e = a;
    e.B = INT_MAX; e.H = INT_MAX; e.Tq = INT_MAX; e.Tk = INT_MAX; e.S = INT_MAX;
    expect("attn overflow", gdn_attention_check_args(&e, b.q, b.k, b.v, b.o, nullptr, 0), GDN_ERR_SHAPE);
  }
  for (int Tq : {1, 4, 81})
    for (int Tk : {81, 961})
      for (int S : {1, 880, 3600}) {
        gdn_attn_desc e = a;
        e.Tq = Tq; e.Tk = Tk; e.S = S; e.H = 20; e.D = 112;
        acc += gdn_attention_workspace_size(&e);
      }

  std::printf("sizes checksum %zu\n", acc);
  std::printf("%s: %d failure(s)\n", failures ? "FAILED" : "ok", failures);
  return failures ? 1 : 0;
}

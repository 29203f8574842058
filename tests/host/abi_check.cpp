// Host-side checks of the planner and the argument validation of the C-ABI
// (isa_layout.cpp), built with g++ -fsanitize=address,undefined and run by
// tests/test_abi_host.py.  No HIP: only the host half of the library.
//
// Checked: every workspace slice of every descriptor of a grid (valid and
// invalid values, contiguous and strided tensors) is 256-byte aligned, in
// order and inside the total; the counts follow the count rule; the
// overlap test of output strides agrees with brute-force enumeration of
// addresses on small shapes; the multiply that replaces the division by H
// in the kernels' head addressing is exact for every head index; random
// descriptors never trip the sanitizers.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <random>
#include <set>
#include <vector>

#include "../../sparse_attention_context_amd/csrc/isa_layout.h"

static int g_fail = 0;
#define CHECK(c)                                                         \
  do {                                                                   \
    if (!(c)) {                                                          \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c); \
      ++g_fail;                                                          \
    }                                                                    \
  } while (0)

static isa_desc base_desc() {
  isa_desc d = {};
  d.B = 1; d.H = 2; d.Ns = 300; d.Nc = 200; d.d = 64; d.b = 16;
  d.rho = 0.5; d.gamma = 0.25; d.dtype = ISA_BF16;
  return d;
}

static int count_rule(double f, int n) {
  double c = ceil(f * (double)n - 1e-9);
  return (int)std::min<double>(n, std::max<double>(0, c));
}

// The work split of the bf16 full route (d = 128 and 64): R row tiles of T key tiles;
// workgroup g of sk_grid takes row tiles g, g + sk_grid, ... whole
// (sk_rounds of them), then range g of the remaining row tiles' units
// u = (Ri - sk_rounds sk_grid) T + t, range g covering [g U / G, (g + 1) U / G)
// for G = sk_G.  By enumeration: every range is non-empty and every
// workgroup meets at most 8 row tiles (the persistent kernel's limit), every
// row tile is covered once (whole or by consecutive parts), a row tile meets
// at most sk_P ranges, the closed form of the range holding a unit agrees
// with a search, the rotated key order of a cut row tile gives every part
// one run of key tiles, and the partial buffers hold the split row tiles'
// sk_P rows.
static void check_stream_k(const isa::Layout& L) {
  const int64_t R = (L.full_rows + isa::kFlashRows - 1) / isa::kFlashRows * L.BH;
  // (d = 64 may leave it off: full_splits equal parts on the first-design kernel)
  const bool on = L.es == 2 && R > 0 && (L.d == 128 || (L.d == 64 && L.sk_grid > 0));
  CHECK(on ? L.sk_grid >= 1 && L.sk_rounds >= 0 && L.sk_P >= 1 && L.sk_P <= isa::kMaxSplits
           : L.sk_grid == 0 && L.sk_G == 0 && L.sk_P == 0);
  if (!on) return;
  const int64_t T = ((int64_t)L.Ns + L.ctx_tok + 63) / 64, R0 = (int64_t)L.sk_rounds * L.sk_grid;
  const int64_t U = (R - R0) * T, G = L.sk_G;
  CHECK(R0 <= R && L.sk_rounds <= 5 && (U > 0) == (G > 0) && G <= L.sk_grid);
  if (L.sk_grid > 100000 || R > 4000000) return;
  auto bound = [&](int64_t g) { return g * U / G; };
  std::vector<int> cover(R, 0), parts(R, 0);
  int max_parts = 0;
  for (int64_t g = 0; g < L.sk_grid; ++g) {
    int items = L.sk_rounds;
    for (int r = 0; r < L.sk_rounds; ++r) cover[r * L.sk_grid + g] += (int)T;
    if (g < G) {
      const int64_t lo = bound(g), hi = bound(g + 1);
      CHECK(hi > lo);
      if (hi <= lo) return;
      items += (int)((hi - 1) / T - lo / T + 1);
      for (int64_t u = lo; u < hi; ++u) ++cover[R0 + u / T];
      for (int64_t r = lo / T; r <= (hi - 1) / T; ++r) max_parts = std::max(max_parts, ++parts[R0 + r]);
    }
    CHECK(items <= 8);
  }
  for (int64_t r = 0; r < R; ++r) CHECK(cover[r] == T);
  CHECK(max_parts <= L.sk_P);
  // range_of(u) = ((u + 1) G + U - 1) / U - 1: the largest g with bound(g) <= u
  for (int64_t g = 0; g < G; g += 1 + G / 64)
    for (int64_t u : {bound(g), bound(g + 1) - 1}) {
      const int64_t rg = ((u + 1) * G + U - 1) / U - 1;
      CHECK(bound(rg) <= u && bound(rg + 1) > u);
    }
  // the rotated key order of a cut row tile (key tile (t - delta) mod T, delta
  // its first inner range boundary): every part is one run of consecutive key
  // tiles inside [0, T), and the parts cover [0, T) once
  auto range_of = [&](int64_t u) { return ((u + 1) * G + U - 1) / U - 1; };
  for (int64_t Rs = 0; G > 0 && Rs < R - R0; ++Rs) {
    const int64_t u0 = Rs * T, gf = range_of(u0), gl = range_of(u0 + T - 1);
    const int64_t delta = (bound(gf) == u0 || gl == gf) ? 0 : bound(gf + 1) - u0;
    std::vector<int> seen(T, 0);
    for (int64_t p = 0; p <= gl - gf; ++p) {
      const int64_t tb = std::max<int64_t>(bound(gf + p) - u0, 0), te = std::min<int64_t>(bound(gf + p + 1) - u0, T);
      const int64_t r = tb >= delta ? tb - delta : tb - delta + T;
      CHECK(r >= 0 && r + (te - tb) <= T);
      for (int64_t k = r; k < r + (te - tb) && k < T; ++k) ++seen[k];
    }
    for (int64_t k = 0; k < T; ++k) CHECK(seen[k] == 1);
    if (Rs > 2000) break;
  }
  if (L.sk_P > 1) {
    CHECK(L.off_part_ml - L.off_part_o >= (size_t)((R - R0) * L.sk_P * isa::kFlashRows * L.d * 2));
    CHECK(L.off_lse - L.off_part_ml >= (size_t)((R - R0) * L.sk_P * isa::kFlashRows * 8));
  }
}

// slices of the forward layout in the order they are carved
static void check_layout(const isa::Layout& L, const isa_desc& D) {
  const size_t offs[] = {L.off_qbar, L.off_kbar, L.off_vbar, L.off_salp, L.off_sal, L.off_kept, L.off_pkhi,
                         L.off_pklo, L.off_pv, L.off_pbias, L.off_ctxrows, L.off_keyrows, L.off_peak, L.off_sh,
                         L.off_fullq, L.off_taylq, L.off_part_o, L.off_part_ml, L.off_lse};
  size_t prev = 0;
  for (size_t i = 0; i < sizeof(offs) / sizeof(offs[0]); ++i) {
    CHECK(offs[i] % isa::kWsAlign == 0);
    CHECK(i == 0 ? offs[i] == 0 : offs[i] > prev);
    prev = offs[i];
  }
  CHECK(L.total > prev && L.total % isa::kWsAlign == 0);
  // the slices that follow each other have room for their contents
  const size_t bh = (size_t)L.BH, d = (size_t)L.d;
  CHECK(L.off_kbar - L.off_qbar >= bh * L.nb_s * d * 4);
  CHECK(L.off_vbar - L.off_kbar >= bh * L.M * d * 4);
  CHECK(L.off_keyrows - L.off_ctxrows >= bh * (size_t)L.ctx_tok * 4);
  CHECK(L.off_peak - L.off_keyrows >= bh * (size_t)L.n_keytab * 4);
  CHECK(L.total - L.off_lse >= bh * (size_t)L.Ns * 4);
  CHECK(L.nb_s == (D.Ns + D.b - 1) / D.b);
  CHECK(L.nb_c == (D.Nc + D.b - 1) / D.b);
  CHECK(L.kc == count_rule(D.rho, L.nb_c));
  CHECK(L.kq == count_rule(D.gamma, L.nb_s));
  CHECK(L.mk_pad % isa::kTileKeys == 0 && L.mk_pad >= L.mk);
  CHECK(L.full_splits >= 1 && L.full_splits <= isa::kMaxSplits);
  CHECK((int64_t)L.n_keytab >= (int64_t)L.Ns + L.ctx_tok && L.n_keytab % isa::kTileKeys == 0);
  check_stream_k(L);
  isa::BwdLayout W;
  if (isa::make_bwd_layout(L, &W) == ISA_OK) {
    CHECK(W.total % isa::kWsAlign == 0 && W.off_rdel < W.total);
    CHECK(W.dkv_splits >= 1 && W.dkv_splits <= 64);
    // the last round of the full-route dK/dV items: cut only when at most
    // half full, into at most kBwdMaxParts ranges of at least one query tile
    const int64_t items = (int64_t)L.BH * ((L.Ns + L.ctx_tok + isa::kBwdKeys - 1) / isa::kBwdKeys);
    CHECK((int64_t)W.kv_rounds * isa::kCUs + W.kv_rest == items);
    CHECK(W.kv_parts == 0 || (W.kv_parts >= 2 && W.kv_parts <= isa::kBwdMaxParts && L.d == 128 &&
                              (int64_t)W.kv_rest * W.kv_parts <= isa::kCUs && W.kv_parts <= W.n_rowtab / 64));
    CHECK(W.off_rrow - W.off_part_kv >= (size_t)W.kv_rest * W.kv_parts * isa::kBwdKeys * L.d * 4);
    // the dQ cut of the last round of row tiles, and room for its partials
    const int64_t rtiles = (int64_t)L.BH * ((L.full_rows + isa::kFlashRows - 1) / isa::kFlashRows);
    CHECK((int64_t)W.dq_rounds * isa::kCUs + W.dq_rest == rtiles);
    CHECK(W.dq_parts == 0 || (W.dq_parts >= 2 && W.dq_parts <= isa::kMaxSplits && L.d == 128 &&
                              (int64_t)W.dq_rest * W.dq_parts <= isa::kCUs));
    CHECK(W.off_part_kv - W.off_part_dq >= (size_t)W.dq_rest * W.dq_parts * isa::kFlashRows * L.d * 4);
  }
  isa::Fp8Layout F;
  if (isa::make_fp8_layout(L, &F) == ISA_OK) CHECK(F.nkp % 64 == 0 && F.off_vs < F.total);
}

// every element address of a [B,H,rows,d] tensor under m is distinct
static bool brute_disjoint(const isa::RowMap& m, int B, int rows, int d) {
  std::set<int64_t> seen;
  for (int x = 0; x < B; ++x)
    for (int h = 0; h < m.H; ++h)
      for (int r = 0; r < rows; ++r)
        for (int e = 0; e < d; ++e)
          if (!seen.insert(x * m.sb + h * m.sh + (int64_t)r * m.sn + e).second) return false;
  return true;
}

int main() {
  // ---- a grid of descriptors, contiguous and strided
  const int Bs[] = {1, 2, 3};
  const int Hs[] = {1, 2, 5};
  const int Nss[] = {1, 37, 256, 1000};
  const int Ncs[] = {0, 23, 256, 700};
  const int ds[] = {64, 128, 96};
  const int bs[] = {1, 16, 64, 200, 256, 257};
  const double fr[] = {0.0, 0.2, 0.25, 1.0, -0.1, 1.5, NAN};
  int n_ok = 0, n_err = 0;
  for (int B : Bs)
    for (int H : Hs)
      for (int Ns : Nss)
        for (int Nc : Ncs)
          for (int d : ds)
            for (int b : bs)
              for (double rho : fr)
                for (int layout = 0; layout < 3; ++layout) {
                  isa_desc D = base_desc();
                  D.B = B; D.H = H; D.Ns = Ns; D.Nc = Nc; D.d = d; D.b = b;
                  D.rho = rho; D.gamma = fr[(b + Ns) % 7]; D.dtype = (Ns + Nc) % 2 ? ISA_F32 : ISA_BF16;
                  const int64_t nk = (int64_t)Ns + Nc;
                  if (layout == 1) {   // [B,N,H,d] views: tokens before heads
                    D.q = {(int64_t)Ns * H * d, d, (int64_t)H * d};
                    D.k = {nk * H * d, d, (int64_t)H * d};
                    D.v = D.k;
                    D.o = D.q;
                  } else if (layout == 2) {   // rows padded by 64 elements
                    D.q = {(int64_t)H * Ns * (d + 64), (int64_t)Ns * (d + 64), d + 64};
                    D.k = {(int64_t)H * nk * (d + 64), nk * (d + 64), d + 64};
                    D.v = D.k;
                    D.o = D.q;
                  }
                  isa::Layout L;
                  const isa_status st = isa::make_layout(&D, &L);
                  size_t ws = 0;
                  CHECK(isa_workspace_size(&D, &ws) == st);
                  if (st == ISA_OK) {
                    ++n_ok;
                    CHECK(ws == L.total);
                    check_layout(L, D);
                    isa_counts c;
                    CHECK(isa_get_counts(&D, &c) == ISA_OK && c.kc == L.kc && c.kq == L.kq);
                    // plan views point inside a workspace of that size
                    if (L.total > (size_t(1) << 20)) continue;
                    std::vector<char> buf(L.total + 256);
                    char* w = (char*)(((uintptr_t)buf.data() + 255) / 256 * 256);
                    isa_plan_view v;
                    CHECK(isa_plan_views(&D, w, L.total, &v) == ISA_OK);
                    CHECK((const char*)v.taylor_q >= w && (const char*)v.taylor_q < w + L.total);
                    CHECK(isa_plan_views(&D, w, L.total - 1, &v) == ISA_ERR_WORKSPACE);
                  } else {
                    ++n_err;
                    const bool bad_arg = !(rho >= 0 && rho <= 1) || !(D.gamma >= 0 && D.gamma <= 1);
                    const bool unsup = d == 96 || b > 256;
                    CHECK(bad_arg ? st == ISA_ERR_INVALID_ARGUMENT : true);
                    CHECK(!bad_arg && unsup ? st == ISA_ERR_UNSUPPORTED : true);
                  }
                }
  CHECK(n_ok > 1000 && n_err > 1000);

  // ---- limits
  {
    isa_desc D = base_desc();
    isa::Layout L;
    D.B = 256; D.H = 256;   // B*H = 65536
    CHECK(isa::make_layout(&D, &L) == ISA_ERR_UNSUPPORTED);
    D.H = 255;
    CHECK(isa::make_layout(&D, &L) == ISA_OK);
    D = base_desc(); D.Ns = (1 << 24) - 100; D.Nc = 100;
    CHECK(isa::make_layout(&D, &L) == ISA_ERR_UNSUPPORTED);
    D.Nc = 99; D.d = 64;
    CHECK(isa::make_layout(&D, &L) == ISA_OK);   // 2^24 - 1 rows of 128 bytes: under 2^31
    D.d = 128;
    CHECK(isa::make_layout(&D, &L) == ISA_ERR_UNSUPPORTED);   // a head of K spans 2^32 bytes
    D = base_desc(); D.reserved = 1;
    CHECK(isa::make_layout(&D, &L) == ISA_ERR_INVALID_ARGUMENT);
    D = base_desc(); D.k = {0, 0, -64};
    CHECK(isa::make_layout(&D, &L) == ISA_ERR_INVALID_ARGUMENT);
    D = base_desc(); D.k = {500 * 2 * 64, 500 * 64, 65};   // rows of 130 bytes: misaligned
    CHECK(isa::make_layout(&D, &L) == ISA_ERR_INVALID_ARGUMENT);
    D = base_desc(); D.k = {500 * 2 * (int64_t)(1 << 23), 500 * (int64_t)(1 << 23), 1 << 23};   // row step 2^24 bytes
    CHECK(isa::make_layout(&D, &L) == ISA_ERR_UNSUPPORTED);
    D = base_desc(); D.o = {300 * 2 * 64, 300 * 64, 32};   // O rows overlap
    CHECK(isa::make_layout(&D, &L) == ISA_ERR_INVALID_ARGUMENT);
    D = base_desc(); D.q = {300 * 2 * 64, 300 * 64, 32};   // Q rows overlap: a valid input
    CHECK(isa::make_layout(&D, &L) == ISA_OK);
    D = base_desc(); D.o = {64, 64, 128};   // heads interleaved with rows: disjoint
    D.H = 2;
    CHECK(isa::make_layout(&D, &L) == ISA_OK);
    D.o = {64, 0, 128};   // both heads on one address range
    CHECK(isa::make_layout(&D, &L) == ISA_ERR_INVALID_ARGUMENT);
  }

  // ---- pointer and workspace checks
  {
    alignas(256) static char mem[1024];
    const void* ok[4] = {mem, mem + 16, mem + 32, mem + 48};
    CHECK(isa::check_tensors(ok, 4) == ISA_OK);
    const void* mis[2] = {mem, mem + 8};
    CHECK(isa::check_tensors(mis, 2) == ISA_ERR_INVALID_ARGUMENT);
    const void* nul[2] = {mem, nullptr};
    CHECK(isa::check_tensors(nul, 2) == ISA_ERR_INVALID_ARGUMENT);
    CHECK(isa::check_workspace(mem, 1024, 1024) == ISA_OK);
    CHECK(isa::check_workspace(mem, 1023, 1024) == ISA_ERR_WORKSPACE);
    CHECK(isa::check_workspace(mem + 16, 1024, 512) == ISA_ERR_WORKSPACE);
    CHECK(isa::check_workspace(nullptr, 1024, 512) == ISA_ERR_INVALID_ARGUMENT);
  }

  // ---- overlap test of output strides against brute force
  {
    std::mt19937 rng(7);
    int agree = 0, disjoint = 0;
    for (int it = 0; it < 4000; ++it) {
      const int B = 1 + rng() % 3, H = 1 + rng() % 3, rows = 1 + rng() % 4, d = 1 + rng() % 4;
      isa::RowMap m = {};
      m.H = H;
      m.sb = rng() % 40;
      m.sh = rng() % 20;
      m.sn = (int32_t)(rng() % 10);
      const bool got = isa::map_disjoint(m, B, rows, d);
      const bool want = brute_disjoint(m, B, rows, d);
      // the test is sufficient (never accepts an overlap); on these small
      // shapes it is also exact for layouts whose strides nest
      CHECK(!got || want);
      agree += got == want;
      disjoint += want;
    }
    printf("overlap test: %d of 4000 layouts disjoint, the check agrees with brute force on %d\n", disjoint, agree);
    CHECK(disjoint > 200 && agree > 3000);
  }

  // ---- head index by multiply: x = (bh * hmul) >> 32 == bh / H for every bh < 2^16
  {
    auto check_H = [&](int H) {
      isa_desc D = base_desc();
      D.B = 1; D.H = H; D.Ns = 16; D.Nc = 0;
      isa::Layout L;
      if (isa::make_layout(&D, &L) != ISA_OK) return;
      for (uint32_t bh = 0; bh < 65536u; ++bh) {
        const uint32_t x = H == 1 ? bh : (uint32_t)(((uint64_t)bh * L.q.hmul) >> 32);
        if (x != bh / (uint32_t)H) {
          CHECK(x == bh / (uint32_t)H);
          return;
        }
      }
    };
    for (int H = 1; H <= 1024; ++H) check_H(H);
    std::mt19937 rng(11);
    for (int i = 0; i < 512; ++i) check_H(1025 + (int)(rng() % 64510));
    check_H(65535);
  }

  // ---- stream-K ranges at large sizes: the video-DiT layer, and layers with
  // enough row tiles that the range count passes the compute-unit count
  {
    const int shapes[][5] = {{1, 24, 17550, 17550, 64}, {1, 64, 200000, 50000, 64}, {2, 40, 60000, 0, 128},
                             {1, 1, 4194000, 4194300, 64}, {3, 7, 5000, 123, 16}};
    for (const auto& sh : shapes)
      for (double gamma : {0.2, 1.0}) {
        isa_desc D = base_desc();
        D.B = sh[0]; D.H = sh[1]; D.Ns = sh[2]; D.Nc = sh[3]; D.b = sh[4]; D.d = 128;
        D.rho = 0.25; D.gamma = gamma;
        isa::Layout L;
        CHECK(isa::make_layout(&D, &L) == ISA_OK);
        check_layout(L, D);
      }
  }

  // ---- random descriptors: no sanitizer finding, errors only as documented
  {
    std::mt19937_64 rng(5);
    for (int it = 0; it < 200000; ++it) {
      isa_desc D;
      uint64_t* p = (uint64_t*)&D;
      for (size_t i = 0; i < sizeof(D) / 8; ++i) p[i] = rng();
      if (it % 2) {   // plausible sizes, random strides
        D.B = 1 + rng() % 4; D.H = 1 + rng() % 64; D.Ns = 1 + rng() % 100000; D.Nc = rng() % 100000;
        D.d = (rng() % 2) ? 64 : 128; D.b = 1 + rng() % 300; D.rho = (rng() % 1001) / 1000.0;
        D.gamma = (rng() % 1001) / 1000.0; D.dtype = rng() % 2; D.reserved = 0;
      }
      size_t ws;
      const isa_status st = isa_workspace_size(&D, &ws);
      CHECK(st == ISA_OK || st == ISA_ERR_INVALID_ARGUMENT || st == ISA_ERR_UNSUPPORTED);
      isa_counts c;
      CHECK(isa_get_counts(&D, &c) == st);
      size_t bws;
      const isa_status sb = isa_backward_workspace_size(&D, &bws);
      CHECK(st != ISA_OK || sb == ISA_OK || sb == ISA_ERR_UNSUPPORTED);
    }
  }

  if (g_fail) {
    fprintf(stderr, "%d checks failed\n", g_fail);
    return 1;
  }
  printf("abi_check ok\n");
  return 0;
}

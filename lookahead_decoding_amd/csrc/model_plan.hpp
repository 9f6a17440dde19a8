// Host-side layout of the layer forward: where each weight tensor sits in the
// caller's weight buffer, the GEMM plans of one layer and the carve-up of the
// forward's workspace.  Pure host code.
#pragma once

#include "attn_plan.hpp"
#include "gemm_plan.hpp"
#include "lopa.h"

namespace lopa {

inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

struct ModelShape {
  int hidden, qkv, hq_d, inter, M;
};

inline ModelShape model_shape(const lopa_dims& d, const lopa_model_dims& md) {
  ModelShape s;
  s.hq_d = d.Hq * d.d;
  s.hidden = s.hq_d;
  s.qkv = (d.Hq + 2 * d.Hkv) * d.d;
  s.inter = md.inter;
  s.M = (d.k_max + 1) * d.B;
  return s;
}

inline lopa_model_layout model_layout(const lopa_dims& d, const lopa_model_dims& md) {
  const ModelShape s = model_shape(d, md);
  const size_t h = static_cast<size_t>(s.hidden);
  lopa_model_layout o{};
  size_t at = 0;
  auto take = [&](size_t elems) {
    const size_t here = at;
    at = align256(at + elems * 2);
    return here;
  };
  o.attn_norm = take(h);
  o.wqkv = take(static_cast<size_t>(s.qkv) * h);
  o.bqkv = take(static_cast<size_t>(s.qkv));
  o.wo = take(h * s.hq_d);
  o.mlp_norm = take(h);
  o.wgu = take(2 * static_cast<size_t>(s.inter) * h);
  o.wd = take(h * s.inter);
  o.layer_stride = at;
  o.layer0 = 0;
  at = o.layer_stride * static_cast<size_t>(md.n_layers);
  o.final_norm = take(h);
  o.embed = take(static_cast<size_t>(d.V) * h);
  o.lm_head = take(static_cast<size_t>(d.V) * h);
  o.total = at;
  return o;
}

// The four projections of one layer, in order: q/k/v, output, gate+up, down.
// Where the shape allows (glu_on), gate+up and its SwiGLU run as one kernel
// over the GluView and write no partial tiles.
struct LayerGemms {
  GemmView qkv, o, gu, down;
  GluView glu;
  bool glu_on;
  size_t partial_bytes() const {
    size_t b = qkv.partial_bytes();
    if (o.partial_bytes() > b) b = o.partial_bytes();
    if (!glu_on && gu.partial_bytes() > b) b = gu.partial_bytes();
    if (down.partial_bytes() > b) b = down.partial_bytes();
    return b;
  }
};

// XCD-aligned stream-K split: G = a * units workgroups, a dividing the K
// chunk count, so workgroup g = a u + j takes K slice j of unit u.  The
// eight XCDs take workgroups round robin (g mod 8), so with a = 8 every XCD
// reads one eighth of the activation's K range and with a = 4 one quarter:
// the slice stays in the XCD's own L2 (the down projection's activation is
// 6 MB at 160 rows, more than one XCD's 4 MB L2, and was fetched from
// memory again and again: 249 MB fetched for a 136 MB weight), and each
// unit's K range is cut into exactly a pieces.  Falls back to the plain
// split when a does not divide the chunk count or a * units exceeds the
// workgroup limit.
inline GemmView aligned_view(int M, int N, int K, int a) {
  const GemmView v = gemm_view(M, N, K);
  if (v.nch % a != 0 || a * v.units > kGemmMaxWorkgroups) return v;
  return gemm_view(M, N, K, a * v.units);
}

// At 129-160 rows (5 branches of 32) the q/k/v and output projections use
// a = 4 and the down projection a = 8.  Measured on the 28-layer 7B forward
// at 5 branches (same box): 5.37 against 5.51 ms for 160 workgroups on q/k/v
// and output with the plain split elsewhere, which in turn beat 256
// workgroups (5.51 against 5.78 ms); gate+up keeps 256 (8 * 148 units would
// exceed the limit, and its 1.15 MB activation fits every L2).
inline LayerGemms layer_gemms(const lopa_dims& d, const lopa_model_dims& md) {
  const ModelShape s = model_shape(d, md);
  LayerGemms g;
  const bool five = s.M > 128 && s.M <= 160;
  g.qkv = five ? aligned_view(s.M, s.qkv, s.hidden, 4) : gemm_view(s.M, s.qkv, s.hidden);
  g.o = five ? aligned_view(s.M, s.hidden, s.hq_d, 4) : gemm_view(s.M, s.hidden, s.hq_d);
  g.gu = gemm_view(s.M, 2 * s.inter, s.hidden);
  g.glu_on = glu_fits(s.M, s.hidden, s.inter);
  g.glu = glu_view(s.M, s.hidden, s.inter);
  g.down = five ? aligned_view(s.M, s.hidden, s.inter, 8) : gemm_view(s.M, s.hidden, s.inter);
  return g;
}

// Workspace of lopa_branch_forward: residual stream x (float32), normed
// activations h (bf16), Q, attention output, MLP activation (bf16), the
// rotary table of the block's positions, GEMM partials and the attention
// call's own workspace.
struct ModelWorkspace {
  size_t x, h, q, ho, act, rope, part, attn, total;
};

inline ModelWorkspace model_workspace(const lopa_dims& d, const lopa_model_dims& md) {
  const ModelShape s = model_shape(d, md);
  const size_t M = static_cast<size_t>(s.M);
  ModelWorkspace w{};
  size_t at = 0;
  auto take = [&](size_t bytes) {
    const size_t here = at;
    at = align256(at + bytes);
    return here;
  };
  w.x = take(M * s.hidden * 4);
  w.h = take(M * s.hidden * 2);
  w.q = take(M * s.hq_d * 2);
  w.ho = take(M * s.hq_d * 2);
  w.act = take(M * s.inter * 2);
  w.rope = take(static_cast<size_t>(d.B) * (d.d / 2) * 8);   // (cos, sin) float pairs
  w.part = take(layer_gemms(d, md).partial_bytes());
  w.attn = take(attn_workspace_bytes(d));
  w.total = at;
  return w;
}

}  // namespace lopa

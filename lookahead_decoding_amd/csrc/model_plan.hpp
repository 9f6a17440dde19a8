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
struct LayerGemms {
  GemmView qkv, o, gu, down;
  size_t partial_bytes() const {
    size_t b = qkv.partial_bytes();
    if (o.partial_bytes() > b) b = o.partial_bytes();
    if (gu.partial_bytes() > b) b = gu.partial_bytes();
    if (down.partial_bytes() > b) b = down.partial_bytes();
    return b;
  }
};

inline LayerGemms layer_gemms(const lopa_dims& d, const lopa_model_dims& md) {
  const ModelShape s = model_shape(d, md);
  LayerGemms g;
  g.qkv = gemm_view(s.M, s.qkv, s.hidden);
  g.o = gemm_view(s.M, s.hidden, s.hq_d);
  g.gu = gemm_view(s.M, 2 * s.inter, s.hidden);
  g.down = gemm_view(s.M, s.hidden, s.inter);
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

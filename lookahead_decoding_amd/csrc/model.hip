// Layer forward of the verification pass: every live branch's block through
// a Qwen2.5/Dream-7B-shaped decoder (RMSNorm, q/k/v projections with bias,
// rotary embedding, branch-isolated attention over the committed prefix,
// output projection, RMSNorm, SwiGLU MLP; residual stream in float32), then
// the final RMSNorm whose rows feed lopa_lmhead_conf.
//
// The news article "上交大 × 华为小艺推出LoPA：7B扩散语言模型单样例1000+ tokens/s！"
// (section "LoPA 的核心设计：前瞻并行与分支验证", stage 并行验证与复用) verifies
// all branches in one forward pass; section 3.3 of "解码效率革命：LoPA如何突破
// 扩散语言模型的并行瓶颈" keeps each branch's attention to the original input and
// its own tokens and computes every branch in one shared matrix multiply;
// section 6 of the same article requires full-sequence attention.  Here the
// branches are rows of one batch: every projection streams its weight once
// for all of them (k_gemm_stream), attention is lopa_branch_attn.
//
// Rounding points (shared with the oracle): the normed activations, Q/K/V
// after bias and rotation, the attention output and the MLP activation are
// rounded once to bf16 (nearest even); projections accumulate in float32
// and are added to the float32 residual stream.
#include "model_plan.hpp"
#include "philox.hpp"

namespace lopa {

int gemm_launch(const GemmView& v, const unsigned short* X, const unsigned short* W, float* P,
                hipStream_t stream);
int glu_launch(const GluView& v, const unsigned short* X, const unsigned short* W,
               unsigned short* act, hipStream_t stream);

// ---------------------------------------------------------------------------
// Synthetic weights
// ---------------------------------------------------------------------------

enum SynthRule { kRuleUniform = 0, kRuleNorm = 1 };

// One thread per 4 consecutive columns of one row: Philox4x32-10 with key
// (seed low, seed high) and counter (col / 4, row, id | layer << 8, 0) gives
// the four words; word j serves column 4 (col / 4) + j.
//   uniform, shift s: ((x >> 8) - 2^23) * 2^(-24 - s), rounded to bf16
//   norm:             1 + ((x >> 27) - 16) * 2^-7 (exact in bf16)
__global__ void __launch_bounds__(256)
k_synth_tensor(unsigned short* __restrict__ out, int rows, int cols, unsigned id,
               unsigned layer, int rule, float scale, unsigned k0, unsigned k1) {
  const int quads = (cols + 3) >> 2;
  const long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<long long>(rows) * quads) return;
  const int row = static_cast<int>(i / quads);
  const int q = static_cast<int>(i - static_cast<long long>(row) * quads);
  const U32x4 r = philox4x32_10(
      U32x4{static_cast<unsigned>(q), static_cast<unsigned>(row), id | (layer << 8), 0u}, k0, k1);
  const unsigned xs[4] = {r.x0, r.x1, r.x2, r.x3};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int col = 4 * q + j;
    if (col >= cols) break;
    float v;
    if (rule == kRuleNorm) {
      v = 1.f + static_cast<float>(static_cast<int>(xs[j] >> 27) - 16) * (1.f / 128.f);
    } else {
      // exact in float32: a multiple of 2^-24 below 1/2 in magnitude
      v = static_cast<float>(static_cast<int>(xs[j] >> 8) - (1 << 23)) * (1.f / 16777216.f);
      v *= scale;   // a power of two: exact
    }
    out[static_cast<size_t>(row) * cols + col] = f32_to_bf16_bits(v);
  }
}

// ---------------------------------------------------------------------------
// Row-wise kernels (one workgroup of kRowThreads threads per activation row:
// at hidden <= 4 * kRowThreads every thread owns one group of four columns,
// so a row's loads are all issued at once)
// ---------------------------------------------------------------------------

constexpr int kRowThreads = 1024;

__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kRowThreads / 64; ++i) s += red[i];
  __syncthreads();
  return s;
}

// h[r] = bf16(x[r] / sqrt(mean(x[r]^2) + eps) * g) for the float32 row x[r]
// this thread has just written (the same thread re-reads its own elements,
// four at a time: hidden is a multiple of 64).
__device__ __forceinline__ void norm_row(const float* __restrict__ xr, float ss, int hidden,
                                         float eps, const unsigned short* __restrict__ g,
                                         unsigned short* __restrict__ hr, float* red) {
  const float tot = block_sum(ss, red);
  const float rs = 1.f / sqrtf(tot / static_cast<float>(hidden) + eps);
  for (int n = 4 * threadIdx.x; n < hidden; n += 4 * kRowThreads) {
    const float4 x = *reinterpret_cast<const float4*>(xr + n);
    const ushort4 gg = *reinterpret_cast<const ushort4*>(g + n);
    ushort4 o;
    o.x = f32_to_bf16_bits(x.x * rs * bf16_bits_to_f32(gg.x));
    o.y = f32_to_bf16_bits(x.y * rs * bf16_bits_to_f32(gg.y));
    o.z = f32_to_bf16_bits(x.z * rs * bf16_bits_to_f32(gg.z));
    o.w = f32_to_bf16_bits(x.w * rs * bf16_bits_to_f32(gg.w));
    *reinterpret_cast<ushort4*>(hr + n) = o;
  }
}

// Embedding of each row's token (the mask token's row where masked) into the
// residual stream, then the first layer's input norm.
__global__ void __launch_bounds__(kRowThreads)
k_embed_norm(int hidden, int V, int mask_id, float eps, const int32_t* __restrict__ tok,
             const unsigned short* __restrict__ E, const unsigned short* __restrict__ g,
             float* __restrict__ x, unsigned short* __restrict__ h) {
  __shared__ float red[kRowThreads / 64];
  const int r = blockIdx.x;
  const int t = tok[r];
  const int e = t == LOPA_MASK_TOKEN ? mask_id : min(max(t, 0), V - 1);
  float* xr = x + static_cast<size_t>(r) * hidden;
  const unsigned short* er = E + static_cast<size_t>(e) * hidden;
  float ss = 0.f;
  for (int n = 4 * threadIdx.x; n < hidden; n += 4 * kRowThreads) {
    const ushort4 ev = *reinterpret_cast<const ushort4*>(er + n);
    const float4 v = make_float4(bf16_bits_to_f32(ev.x), bf16_bits_to_f32(ev.y),
                                 bf16_bits_to_f32(ev.z), bf16_bits_to_f32(ev.w));
    *reinterpret_cast<float4*>(xr + n) = v;
    ss = fmaf(v.x, v.x, ss);
    ss = fmaf(v.y, v.y, ss);
    ss = fmaf(v.z, v.z, ss);
    ss = fmaf(v.w, v.w, ss);
  }
  norm_row(xr, ss, hidden, eps, g, h + static_cast<size_t>(r) * hidden, red);
}

// x[r] += (the projection's row r, summed from its partial tiles), then the
// next norm of the row.
__global__ void __launch_bounds__(kRowThreads)
k_residual_norm(GemmView v, const float* __restrict__ P, float eps,
                const unsigned short* __restrict__ g, float* __restrict__ x,
                unsigned short* __restrict__ h) {
  __shared__ float red[kRowThreads / 64];
  __shared__ unsigned char tab[kSlotTableMax];
  v.load_slots(tab);
  __syncthreads();
  const int r = blockIdx.x;
  const int hidden = v.N;
  float* xr = x + static_cast<size_t>(r) * hidden;
  float ss = 0.f;
  for (int n = 4 * threadIdx.x; n < hidden; n += 4 * kRowThreads) {
    float4 y = *reinterpret_cast<const float4*>(xr + n);
    const float4 d = v.sum4<8>(P, tab, r, n);
    y.x += d.x;
    y.y += d.y;
    y.z += d.z;
    y.w += d.w;
    *reinterpret_cast<float4*>(xr + n) = y;
    ss = fmaf(y.x, y.x, ss);
    ss = fmaf(y.y, y.y, ss);
    ss = fmaf(y.z, y.z, ss);
    ss = fmaf(y.w, y.w, ss);
  }
  norm_row(xr, ss, hidden, eps, g, h + static_cast<size_t>(r) * hidden, red);
}

// Rotary table of the block's positions: (cos, sin) of (L + p) * theta^(-2i/d)
// for p < B, i < d/2, evaluated in double and rounded to float once.
__global__ void __launch_bounds__(256)
k_rope_table(int B, int L, int d, double log2_theta, float2* __restrict__ tab) {
  const int half = d >> 1;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= B * half) return;
  const int p = idx / half, i = idx - p * half;
  const double ang =
      static_cast<double>(L + p) * exp2(-2.0 * static_cast<double>(i) / d * log2_theta);
  tab[idx] = make_float2(static_cast<float>(cos(ang)), static_cast<float>(sin(ang)));
}

// q/k/v of row r: projection + bias; q and k turned by the rotary table
// (pairs (i, i + d/2)); all three rounded to bf16.  One thread per (row,
// head, 4 consecutive i < d/2); heads 0..Hq-1 are q's, then k's, then v's.
// d is a multiple of 8.
__global__ void __launch_bounds__(256)
k_qkv_epilogue(GemmView v, const float* __restrict__ P, int B, int Hq, int Hkv, int d,
               const float2* __restrict__ rope, const unsigned short* __restrict__ bias,
               unsigned short* __restrict__ Q, unsigned short* __restrict__ K,
               unsigned short* __restrict__ Vo) {
  __shared__ unsigned char tab[kSlotTableMax];
  v.load_slots(tab);
  __syncthreads();
  const int half = d >> 1, quads = half >> 2;
  const int heads = Hq + 2 * Hkv;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= v.M * heads * quads) return;
  const int i0 = 4 * (idx % quads);
  const int hh = (idx / quads) % heads;
  const int r = idx / (quads * heads);
  const int ni = hh * d + i0, nj = ni + half;
  const float4 pa = v.sum4<8>(P, tab, r, ni), pb = v.sum4<8>(P, tab, r, nj);
  float a[4] = {pa.x, pa.y, pa.z, pa.w}, b[4] = {pb.x, pb.y, pb.z, pb.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    a[j] += bf16_bits_to_f32(bias[ni + j]);
    b[j] += bf16_bits_to_f32(bias[nj + j]);
  }
  if (hh < Hq + Hkv) {
    const float2* cs = rope + (r % B) * half + i0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float c = cs[j].x, s = cs[j].y;
      const float a2 = a[j] * c - b[j] * s;
      const float b2 = b[j] * c + a[j] * s;
      a[j] = a2;
      b[j] = b2;
    }
  }
  unsigned short* dst;
  size_t base;
  if (hh < Hq) {
    dst = Q;
    base = (static_cast<size_t>(r) * Hq + hh) * d;
  } else if (hh < Hq + Hkv) {
    dst = K;
    base = (static_cast<size_t>(r) * Hkv + (hh - Hq)) * d;
  } else {
    dst = Vo;
    base = (static_cast<size_t>(r) * Hkv + (hh - Hq - Hkv)) * d;
  }
  ushort4 oa, ob;
  oa.x = f32_to_bf16_bits(a[0]); oa.y = f32_to_bf16_bits(a[1]);
  oa.z = f32_to_bf16_bits(a[2]); oa.w = f32_to_bf16_bits(a[3]);
  ob.x = f32_to_bf16_bits(b[0]); ob.y = f32_to_bf16_bits(b[1]);
  ob.z = f32_to_bf16_bits(b[2]); ob.w = f32_to_bf16_bits(b[3]);
  *reinterpret_cast<ushort4*>(dst + base + i0) = oa;
  *reinterpret_cast<ushort4*>(dst + base + i0 + half) = ob;
}

// act[r][j..j+3] = bf16(silu(gate) * up), gate = columns j.. and up = columns
// inter + j.. of the gate/up projection (inter is a multiple of 64).
__global__ void __launch_bounds__(256)
k_swiglu(GemmView v, const float* __restrict__ P, int inter, unsigned short* __restrict__ act) {
  __shared__ unsigned char tab[kSlotTableMax];
  v.load_slots(tab);
  __syncthreads();
  const int q4 = inter >> 2;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= v.M * q4) return;
  const int r = idx / q4;
  const int j = 4 * (idx - r * q4);
  const float4 gt = v.sum4(P, tab, r, j);
  const float4 up = v.sum4(P, tab, r, inter + j);
  ushort4 o;
  o.x = f32_to_bf16_bits(gt.x / (1.f + expf(-gt.x)) * up.x);
  o.y = f32_to_bf16_bits(gt.y / (1.f + expf(-gt.y)) * up.y);
  o.z = f32_to_bf16_bits(gt.z / (1.f + expf(-gt.z)) * up.z);
  o.w = f32_to_bf16_bits(gt.w / (1.f + expf(-gt.w)) * up.w);
  *reinterpret_cast<ushort4*>(act + static_cast<size_t>(r) * inter + j) = o;
}

// Copy of the winner's block K/V slot of every layer to the prefix rows
// at .. at+B-1 of that layer.
template <typename T>
__global__ void __launch_bounds__(256)
k_model_commit(int n, int nb_max, int layers, size_t kb_layer, size_t kp_layer,
               const int32_t* __restrict__ winner, const T* __restrict__ Kb,
               const T* __restrict__ Vb, T* __restrict__ Kp, T* __restrict__ Vp) {
  const int wsel = min(max(*winner, 0), nb_max - 1);
  const long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<long long>(n) * layers) return;
  const int l = static_cast<int>(i / n);
  const int e = static_cast<int>(i - static_cast<long long>(l) * n);
  const size_t src = l * kb_layer + static_cast<size_t>(wsel) * n + e;
  Kp[l * kp_layer + e] = Kb[src];
  Vp[l * kp_layer + e] = Vb[src];
}

}  // namespace lopa

// ---------------------------------------------------------------------------
// Entry points
// ---------------------------------------------------------------------------

static int check_model(const lopa_dims* d, const lopa_model_dims* md) {
  int st = lopa_check_dims(d);
  if (st != LOPA_OK) return st;
  if (!md) return LOPA_ERR_INVALID;
  if (md->n_layers < 1 || md->n_layers > 1024 || md->inter < 1 || md->inter > (1 << 20))
    return LOPA_ERR_INVALID;
  if (md->mask_id < 0 || md->mask_id >= d->V) return LOPA_ERR_INVALID;
  if (!(md->rope_theta > 1.f) || !(md->rms_eps >= 0.f)) return LOPA_ERR_INVALID;
  if (d->dtype != LOPA_BF16) return LOPA_ERR_UNSUPPORTED;
  const lopa::ModelShape s = lopa::model_shape(*d, *md);
  if (s.hidden % 64 != 0 || s.inter % 64 != 0 || d->d % 8 != 0) return LOPA_ERR_UNSUPPORTED;
  // every projection's weight and the embedding rows addressed by 32-bit offsets
  const long long kmax = s.inter > s.hidden ? s.inter : s.hidden;
  const long long nmax = 2LL * s.inter > s.qkv ? 2LL * s.inter : s.qkv;
  if (nmax * kmax * 2 >= (1LL << 31) || static_cast<long long>(s.M) * kmax * 2 >= (1LL << 31))
    return LOPA_ERR_UNSUPPORTED;
  // every projection's units fit the consumers' slot tables
  const lopa::LayerGemms gm = lopa::layer_gemms(*d, *md);
  // (gate+up has no partial tiles where k_gemm_glu serves it)
  const bool gu_parts = !gm.glu_on;
  if (gm.qkv.units > lopa::kSlotTableMax || gm.o.units > lopa::kSlotTableMax ||
      (gu_parts && gm.gu.units > lopa::kSlotTableMax) || gm.down.units > lopa::kSlotTableMax)
    return LOPA_ERR_UNSUPPORTED;
  // the consumers' slot table holds one byte per unit
  if (gm.qkv.smax > 255 || gm.o.smax > 255 || (gu_parts && gm.gu.smax > 255) ||
      gm.down.smax > 255)
    return LOPA_ERR_UNSUPPORTED;
  return LOPA_OK;
}

extern "C" int lopa_model_layout_of(const lopa_dims* dims, const lopa_model_dims* md,
                                    lopa_model_layout* out) {
  int st = check_model(dims, md);
  if (st != LOPA_OK) return st;
  if (!out) return LOPA_ERR_INVALID;
  *out = lopa::model_layout(*dims, *md);
  return LOPA_OK;
}

extern "C" int lopa_model_workspace_bytes(const lopa_dims* dims, const lopa_model_dims* md,
                                          size_t* bytes) {
  int st = check_model(dims, md);
  if (st != LOPA_OK) return st;
  if (!bytes) return LOPA_ERR_INVALID;
  *bytes = lopa::model_workspace(*dims, *md).total;
  return LOPA_OK;
}

// fan-in shift: the integer nearest to log2(sqrt(K / 12)), so that the
// uniform weights have standard deviation about 1 / sqrt(K)
static int fan_in_shift(int K) {
  return static_cast<int>(floor(0.5 * log2(static_cast<double>(K) / 12.0) + 0.5));
}

extern "C" int lopa_model_synth(const lopa_dims* dims, const lopa_model_dims* md, uint64_t seed,
                                void* weights, void* Kp, void* Vp, size_t kv_layer_rows,
                                hipStream_t stream) {
  using namespace lopa;
  int st = check_model(dims, md);
  if (st != LOPA_OK) return st;
  if (!weights || kv_layer_rows < static_cast<size_t>(dims->L)) return LOPA_ERR_INVALID;
  if (dims->L > 0 && (!Kp || !Vp)) return LOPA_ERR_INVALID;
  const ModelShape s = model_shape(*dims, *md);
  const lopa_model_layout lay = model_layout(*dims, *md);
  unsigned char* wb = static_cast<unsigned char*>(weights);
  const unsigned k0 = static_cast<unsigned>(seed), k1 = static_cast<unsigned>(seed >> 32);
  auto gen = [&](size_t off, int rows, int cols, unsigned id, unsigned layer, int rule,
                 int shift) {
    const long long n = static_cast<long long>(rows) * ((cols + 3) / 4);
    if (n == 0) return;
    const float scale = ldexpf(1.f, -shift);
    hipLaunchKernelGGL(k_synth_tensor, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0,
                       stream, reinterpret_cast<unsigned short*>(wb + off), rows, cols, id, layer,
                       rule, scale, k0, k1);
  };
  const int sh_hidden = fan_in_shift(s.hidden), sh_hqd = fan_in_shift(s.hq_d),
            sh_inter = fan_in_shift(s.inter);
  for (int l = 0; l < md->n_layers; ++l) {
    const size_t b = lay.layer0 + static_cast<size_t>(l) * lay.layer_stride;
    gen(b + lay.attn_norm, 1, s.hidden, 0, l, kRuleNorm, 0);
    gen(b + lay.wqkv, s.qkv, s.hidden, 1, l, kRuleUniform, sh_hidden);
    gen(b + lay.bqkv, 1, s.qkv, 2, l, kRuleUniform, 2);
    gen(b + lay.wo, s.hidden, s.hq_d, 3, l, kRuleUniform, sh_hqd);
    gen(b + lay.mlp_norm, 1, s.hidden, 4, l, kRuleNorm, 0);
    gen(b + lay.wgu, 2 * s.inter, s.hidden, 5, l, kRuleUniform, sh_hidden);
    gen(b + lay.wd, s.hidden, s.inter, 6, l, kRuleUniform, sh_inter);
  }
  gen(lay.final_norm, 1, s.hidden, 7, 0, kRuleNorm, 0);
  gen(lay.embed, dims->V, s.hidden, 8, 0, kRuleUniform, 1);
  // the LM head four times wider than fan-in scaling: logits of spread ~4,
  // like the trained model's, so confidences are not all near 1 / V
  gen(lay.lm_head, dims->V, s.hidden, 9, 0, kRuleUniform, sh_hidden - 2);
  const int kvc = dims->Hkv * dims->d;
  const size_t kv_layer_bytes = kv_layer_rows * kvc * 2;
  for (int l = 0; l < md->n_layers && dims->L > 0; ++l) {
    // prefix keys and values: uniform on (-1, 1)
    hipLaunchKernelGGL(k_synth_tensor, dim3(static_cast<unsigned>(
                           (static_cast<long long>(dims->L) * ((kvc + 3) / 4) + 255) / 256)),
                       dim3(256), 0, stream,
                       reinterpret_cast<unsigned short*>(static_cast<unsigned char*>(Kp) +
                                                         l * kv_layer_bytes),
                       dims->L, kvc, 10u, static_cast<unsigned>(l), static_cast<int>(kRuleUniform),
                       2.f, k0, k1);
    hipLaunchKernelGGL(k_synth_tensor, dim3(static_cast<unsigned>(
                           (static_cast<long long>(dims->L) * ((kvc + 3) / 4) + 255) / 256)),
                       dim3(256), 0, stream,
                       reinterpret_cast<unsigned short*>(static_cast<unsigned char*>(Vp) +
                                                         l * kv_layer_bytes),
                       dims->L, kvc, 11u, static_cast<unsigned>(l), static_cast<int>(kRuleUniform),
                       2.f, k0, k1);
  }
  LOPA_LAUNCH_CHECK();
  return LOPA_OK;
}

extern "C" int lopa_branch_forward(const lopa_dims* dims, const lopa_model_dims* md,
                                   const void* weights, const void* Kp, const void* Vp,
                                   size_t kv_layer_rows, const int32_t* br_tok, const int32_t* nb,
                                   void* Kb, void* Vb, void* H, void* ws, size_t ws_bytes,
                                   hipStream_t stream) {
  using namespace lopa;
  int st = check_model(dims, md);
  if (st != LOPA_OK) return st;
  if (!weights || !br_tok || !nb || !Kb || !Vb || !H) return LOPA_ERR_INVALID;
  if (kv_layer_rows < static_cast<size_t>(dims->L)) return LOPA_ERR_INVALID;
  if (dims->L > 0 && (!Kp || !Vp)) return LOPA_ERR_INVALID;
  const ModelWorkspace wsl = model_workspace(*dims, *md);
  if (!ws || ws_bytes < wsl.total) return LOPA_ERR_WORKSPACE;
  const ModelShape s = model_shape(*dims, *md);
  const lopa_model_layout lay = model_layout(*dims, *md);
  const LayerGemms gm = layer_gemms(*dims, *md);
  const unsigned char* wb = static_cast<const unsigned char*>(weights);
  auto wt = [&](size_t off) { return reinterpret_cast<const unsigned short*>(wb + off); };
  unsigned char* w = static_cast<unsigned char*>(ws);
  float* x = reinterpret_cast<float*>(w + wsl.x);
  unsigned short* h = reinterpret_cast<unsigned short*>(w + wsl.h);
  unsigned short* q = reinterpret_cast<unsigned short*>(w + wsl.q);
  unsigned short* ho = reinterpret_cast<unsigned short*>(w + wsl.ho);
  unsigned short* act = reinterpret_cast<unsigned short*>(w + wsl.act);
  float* P = reinterpret_cast<float*>(w + wsl.part);
  float2* rope = reinterpret_cast<float2*>(w + wsl.rope);
  void* aws = w + wsl.attn;
  const size_t aws_bytes = wsl.total - wsl.attn;
  const int M = s.M;
  const size_t kv_rows_elems = static_cast<size_t>(dims->Hkv) * dims->d;
  const size_t kp_layer = kv_layer_rows * kv_rows_elems;            // elements
  const size_t kb_layer = static_cast<size_t>(M) * kv_rows_elems;   // elements
  const double log2_theta = log2(static_cast<double>(md->rope_theta));
  const int heads = dims->Hq + 2 * dims->Hkv;
  const long long qkv_threads = static_cast<long long>(M) * heads * (dims->d / 8);

  const int nrope = dims->B * (dims->d / 2);
  hipLaunchKernelGGL(k_rope_table, dim3((nrope + 255) / 256), dim3(256), 0, stream, dims->B,
                     dims->L, dims->d, log2_theta, rope);
  hipLaunchKernelGGL(k_embed_norm, dim3(M), dim3(kRowThreads), 0, stream, s.hidden, dims->V, md->mask_id,
                     md->rms_eps, br_tok, wt(lay.embed), wt(lay.layer0 + lay.attn_norm), x, h);
  LOPA_LAUNCH_CHECK();
  for (int l = 0; l < md->n_layers; ++l) {
    const size_t lb = lay.layer0 + static_cast<size_t>(l) * lay.layer_stride;
    unsigned short* kb = static_cast<unsigned short*>(Kb) + l * kb_layer;
    unsigned short* vb = static_cast<unsigned short*>(Vb) + l * kb_layer;
    // attention block
    if ((st = gemm_launch(gm.qkv, h, wt(lb + lay.wqkv), P, stream)) != LOPA_OK) return st;
    hipLaunchKernelGGL(k_qkv_epilogue, dim3(static_cast<unsigned>((qkv_threads + 255) / 256)),
                       dim3(256), 0, stream, gm.qkv, P, dims->B, dims->Hq, dims->Hkv, dims->d,
                       rope, wt(lb + lay.bqkv), q, kb, vb);
    LOPA_LAUNCH_CHECK();
    const unsigned short* kp =
        dims->L > 0 ? static_cast<const unsigned short*>(Kp) + l * kp_layer : nullptr;
    const unsigned short* vp =
        dims->L > 0 ? static_cast<const unsigned short*>(Vp) + l * kp_layer : nullptr;
    if ((st = lopa_branch_attn(dims, kp ? kp : kb, vp ? vp : vb, q, kb, vb, nb, ho, aws,
                               aws_bytes, stream)) != LOPA_OK)
      return st;
    if ((st = gemm_launch(gm.o, ho, wt(lb + lay.wo), P, stream)) != LOPA_OK) return st;
    hipLaunchKernelGGL(k_residual_norm, dim3(M), dim3(kRowThreads), 0, stream, gm.o, P, md->rms_eps,
                       wt(lb + lay.mlp_norm), x, h);
    LOPA_LAUNCH_CHECK();
    // MLP block
    if (gm.glu_on) {
      if ((st = glu_launch(gm.glu, h, wt(lb + lay.wgu), act, stream)) != LOPA_OK) return st;
    } else {
      if ((st = gemm_launch(gm.gu, h, wt(lb + lay.wgu), P, stream)) != LOPA_OK) return st;
      const long long na = static_cast<long long>(M) * (s.inter / 4);
      hipLaunchKernelGGL(k_swiglu, dim3(static_cast<unsigned>((na + 255) / 256)), dim3(256), 0,
                         stream, gm.gu, P, s.inter, act);
      LOPA_LAUNCH_CHECK();
    }
    if ((st = gemm_launch(gm.down, act, wt(lb + lay.wd), P, stream)) != LOPA_OK) return st;
    const bool last = l + 1 == md->n_layers;
    const unsigned short* gnext =
        last ? wt(lay.final_norm) : wt(lb + lay.layer_stride + lay.attn_norm);
    hipLaunchKernelGGL(k_residual_norm, dim3(M), dim3(kRowThreads), 0, stream, gm.down, P, md->rms_eps,
                       gnext, x, last ? static_cast<unsigned short*>(H) : h);
    LOPA_LAUNCH_CHECK();
  }
  return LOPA_OK;
}

extern "C" int lopa_model_commit(const lopa_dims* dims, const lopa_model_dims* md,
                                 const int32_t* winner, const void* Kb, const void* Vb, void* Kp,
                                 void* Vp, size_t kv_layer_rows, int32_t at, hipStream_t stream) {
  using namespace lopa;
  int st = check_model(dims, md);
  if (st != LOPA_OK) return st;
  if (!winner || !Kb || !Vb || !Kp || !Vp || at < 0) return LOPA_ERR_INVALID;
  if (static_cast<size_t>(at) + dims->B > kv_layer_rows) return LOPA_ERR_INVALID;
  const int n = dims->B * dims->Hkv * dims->d;
  const size_t kb_layer = static_cast<size_t>(dims->k_max + 1) * n;
  const size_t kp_layer = kv_layer_rows * dims->Hkv * dims->d;
  const size_t row0 = static_cast<size_t>(at) * dims->Hkv * dims->d;
  const long long tot = static_cast<long long>(n) * md->n_layers;
  hipLaunchKernelGGL(k_model_commit<unsigned short>, dim3(static_cast<unsigned>((tot + 255) / 256)),
                     dim3(256), 0, stream, n, dims->k_max + 1, md->n_layers, kb_layer, kp_layer,
                     winner, static_cast<const unsigned short*>(Kb),
                     static_cast<const unsigned short*>(Vb), static_cast<unsigned short*>(Kp) + row0,
                     static_cast<unsigned short*>(Vp) + row0);
  LOPA_LAUNCH_CHECK();
  return LOPA_OK;
}

// The GPT2 training step as tile tasks (model level of the C ABI).
//
// The pith.science review of NNTile ("What carries the argument") states the
// recipe this file follows: split every tensor into tiles along all axes and
// express every layer -- embedding, linear, layer norm, softmax/attention,
// cross-entropy and the Adam update -- as tasks on a few tiles, forward and
// backward, so that one training iteration is a single graph of small tasks.
// The NNTile README ("Minimal working GPT example") supplies the tile flags
// (batch/minibatch, seq, embd, inner and head tiles; seq, head and batch
// tiles divide their axis, embd and inner tiles need not) and the optimiser
// (fused AdamW, eps 1e-8, weight decay 0.1, lr 3e-4, mean loss).
//
// Model form (readings of what the pages leave open): pre-LN GPT2 blocks,
// GELU (tanh) MLP, LayerNorm eps 1e-5 with biased variance, biases on every
// linear layer, causal attention scaled by 1/sqrt(head_dim), LM head tied to
// the token embedding, no dropout, one AdamW group with decay on every
// parameter.
//
// The same file builds the LLaMA-style model (tt_llama_create; the README's
// notebook list names LLaMa as the second model, and the review's
// "Editorial extensions" notes that the tile tasks assemble other
// architectures): pre-RMSNorm blocks, rotary embedding of q and k, a SwiGLU
// MLP, no biases, no position table and an untied head, with the embedding,
// head, loss, optimiser and residency of the GPT2 step unchanged.
//
// Every task below names the tiles it reads and writes; the executor infers
// the ordering. Submission order is the program order of the untiled step:
// embedding, blocks, final LN, head, loss, then the backward in reverse,
// with each parameter's AdamW tasks right after the backward of its layer.
#include <cmath>
#include <cstring>
#include <memory>

#include "tasks.hpp"

using namespace tt;

namespace {

struct BlockT {
  tt_tensor *h_in, *ln1, *n1, *q, *k, *v, *o, *lse, *h_mid, *ln2, *n2, *u, *g;
  tt_tensor* a;  // LLaMA: n2 W_gate (u holds n2 W_up, g the gated product)
};

}  // namespace

struct tt_gpt2 {
  tt_ctx* ctx = nullptr;
  tt_gpt2_config c{};
  tt_gpt2_tiles t{};
  int param_home = TT_HOME_DEVICE;
  // tile grid sizes
  int64_t nb = 0, ns = 0, ntok = 0, NE = 0, NI = 0, NH = 0, NV = 0, rows = 0, hd = 0;
  std::vector<tt_tensor*> P, G, M, Vv;  // parameter, gradient, moments (param_specs order)
  std::vector<tt_tensor*> owned;        // every tensor to destroy
  // activations
  tt_tensor *tokens = nullptr, *ids = nullptr, *labels = nullptr, *sorted = nullptr, *perm = nullptr;
  std::vector<BlockT> blk;
  tt_tensor *h_last = nullptr, *lnf = nullptr, *nf = nullptr, *z = nullptr;
  tt_tensor *ml = nullptr, *ce_parts = nullptr;
  tt_tensor *ce_lse = nullptr, *row_loss = nullptr, *loss = nullptr;
  tt_tensor *dnf = nullptr, *dh = nullptr, *dgu = nullptr, *dn = nullptr, *dO = nullptr, *dq = nullptr,
            *dk = nullptr, *dv = nullptr, *Dv = nullptr;
  tt_tensor *step = nullptr, *bc = nullptr;
  int64_t last_tasks = 0;
  // graph replay of the whole step (tt_gpt2_set_replay): the captured graph
  // and the arguments it was captured with
  bool replay = false;
  hipGraphExec_t graph = nullptr;
  const int32_t* graph_tokens = nullptr;
  tt_adamw_hparams graph_hp{};
  int graph_update = 0;
  int64_t graph_tasks = 0;
  int64_t graph_ws_gen = -1;
  int64_t updates = 0;  // AdamW iterations submitted (warm-up schedule)

  bool llama = false;         // LLaMA-style blocks (tt_llama_create)
  tt_tensor* rope = nullptr;  // LLaMA: rotary cos/sin table [seq, head_dim]

  enum { WTE = 0, WPE = 1 };
  int pidx(int layer, int which) const { return 2 + 12 * layer + which; }
  int lnf_g() const { return 2 + 12 * c.n_layer; }
  // LLaMA parameter indices: wte, 7 per block, norm_f_g, w_head
  int lidx(int layer, int which) const { return 1 + 7 * layer + which; }
  int norm_f() const { return 1 + 7 * c.n_layer; }
  int head_w() const { return llama ? 2 + 7 * c.n_layer : 0; }
};

namespace {

enum { LN1G, LN1B, WQKV, BQKV, WO, BO, LN2G, LN2B, WFC, BFC, WP, BP };
enum { ANORM, LQKV, LWO, MNORM, LGATE, LUP, LDOWN };  // LLaMA block parameters

int mk(tt_gpt2* g, tt_tensor** out, const char* name, std::initializer_list<int64_t> shape,
       std::initializer_list<int64_t> tile, int split, int dtype = TT_F32, int home = TT_HOME_DEVICE) {
  std::vector<int64_t> s(shape), t(tile);
  int rc = tensor_create(g->ctx, (int)s.size(), s.data(), t.data(), dtype, home, split, name, out);
  if (rc == TT_OK) g->owned.push_back(*out);
  return rc;
}

// tile lin helpers
int64_t L(tt_tensor* t, std::initializer_list<int64_t> idx) {
  int64_t a[TT_MAX_DIMS] = {};
  int i = 0;
  for (int64_t v : idx) a[i++] = v;
  return t->lin(a);
}
float* F(tt_tensor* t, int64_t lin) { return (float*)t->dev(lin); }
const int32_t* I32(tt_tensor* t, int64_t lin) { return (const int32_t*)t->dev(lin); }

struct Gemm {
  int ta = 0, tb = 0;
  float alpha = 1.f, beta = 0.f;
  TileRef A, B, C;
  int epi = TT_EPI_NONE;
  TileRef bias, res, aux;
};

TileArg ta(const TileRef& r) { return TileArg{r.t, r.lin}; }

int submit_gemm(tt_ctx* ctx, const char* label, const Gemm& q) {
  TileArg T[6] = {ta(q.A), ta(q.B), ta(q.C)};
  int n = 3;
  if (q.epi & TT_EPI_BIAS) T[n++] = ta(q.bias);
  if (q.epi & TT_EPI_RES) T[n++] = ta(q.res);
  if (q.epi & (TT_EPI_GELU | TT_EPI_GELU_BWD)) T[n++] = ta(q.aux);
  const tt_op_gemm sc{q.ta, q.tb, q.epi, q.alpha, q.beta, 1};
  return submit_op(ctx, TT_OP_GEMM, T, n, &sc, sizeof(sc), label, false);
}

// Independent products (the tied head's per-vocab-tile GEMMs) as
// multi-tile tasks over tile_gemm_batch: consecutive products that share
// transposes, scalars and K form one task (up to 96 products and 1 GiB of
// output tiles, so the grouping depends on the tiling only; sizes and
// leading dimensions may differ, e.g. the ragged last vocab tile). Each
// task reads its A and B tiles and writes (beta == 0) or updates its C
// tiles. With `split`, the task may split K over its stream's workspace
// (few, tall products: the attention weight gradients).
int submit_gemm_batch(tt_ctx* ctx, const char* label, const std::vector<Gemm>& qs, bool split = false) {
  constexpr size_t kMaxProducts = 96;
  constexpr int64_t kMaxBytes = int64_t(1) << 30;
  struct Shape {
    int64_t m, n, k, lda, ldb, ldc;
  };
  auto shape_of = [](const Gemm& q) {
    int64_t ar, ac, br, bc, cr, cc;
    q.A.t->mat(q.A.lin, &ar, &ac);
    q.B.t->mat(q.B.lin, &br, &bc);
    q.C.t->mat(q.C.lin, &cr, &cc);
    return Shape{q.ta ? ac : ar, q.tb ? br : bc, q.ta ? ar : ac, ac, bc, cc};
  };
  size_t i = 0;
  while (i < qs.size()) {
    const Gemm& q0 = qs[i];
    std::vector<Shape> sh = {shape_of(q0)};
    if (q0.epi != TT_EPI_NONE) {
      if (int rc = submit_gemm(ctx, label, q0)) return rc;
      ++i;
      continue;
    }
    int64_t bytes = sh[0].m * sh[0].n * (int64_t)sizeof(float);
    size_t j = i + 1;
    while (j < qs.size() && j - i < kMaxProducts) {
      const Gemm& q = qs[j];
      const Shape s1 = shape_of(q);
      const int64_t b1 = s1.m * s1.n * (int64_t)sizeof(float);
      if (q.ta != q0.ta || q.tb != q0.tb || q.alpha != q0.alpha || q.beta != q0.beta || q.epi != TT_EPI_NONE ||
          s1.k != sh[0].k || bytes + b1 > kMaxBytes)
        break;
      sh.push_back(s1);
      bytes += b1;
      ++j;
    }
    std::vector<TileArg> T;
    for (size_t u = i; u < j; ++u) {
      T.push_back(ta(qs[u].A));
      T.push_back(ta(qs[u].B));
      T.push_back(ta(qs[u].C));
    }
    const tt_op_gemm sc{q0.ta, q0.tb, TT_EPI_NONE, q0.alpha, q0.beta, split ? 1 : 0};
    int rc = submit_op(ctx, TT_OP_GEMM_BATCH, T.data(), (int)T.size(), &sc, sizeof(sc), label, false);
    if (rc) return rc;
    i = j;
  }
  return TT_OK;
}

// C = sum_t A_t B_t^T over the (A, B) tile pairs as one task and one long-K
// launch (tile_gemm_ksum with B transposed): a linear layer's input
// gradient summed over the tiles of its output axis, instead of a chain of
// accumulating GEMMs that each read and write C. A single pair is an
// ordinary tile_gemm task.
int submit_ksum_tb(tt_ctx* ctx, const char* label, TileRef C, const std::vector<TileRef>& As,
                   const std::vector<TileRef>& Bs) {
  if (As.size() == 1) {
    Gemm q;
    q.tb = 1;
    q.A = As[0];
    q.B = Bs[0];
    q.C = C;
    return submit_gemm(ctx, label, q);
  }
  std::vector<TileArg> T = {ta(C)};
  for (size_t u = 0; u < As.size(); ++u) {
    T.push_back(ta(As[u]));
    T.push_back(ta(Bs[u]));
  }
  const tt_op_gemm sc{0, 1, TT_EPI_NONE, 1.f, 0.f, 1};
  return submit_op(ctx, TT_OP_GEMM_KSUM, T.data(), (int)T.size(), &sc, sizeof(sc), label, false);
}

// C = epilogue(sum_t A_t op(B_t)) over the tiles of a linear layer's
// contraction axis as one task: one long-K launch (tile_gemm_ksum_ex) reads
// and writes C once and runs one prologue and epilogue per output block,
// against one per contraction tile for a chain of accumulating GEMMs
// (wide model, MLP input layer 4096 x 8192 x 4 x 2048: 75.5 -> 82.0 % of the
// fp32 peak, measured). A single pair is an ordinary GEMM task.
int submit_ksum(tt_ctx* ctx, const char* label, int tb, TileRef C, const std::vector<TileRef>& As,
                const std::vector<TileRef>& Bs, int epi = TT_EPI_NONE, TileRef bias = {}, TileRef res = {},
                TileRef aux = {}) {
  if (As.size() == 1) {
    Gemm q;
    q.tb = tb;
    q.A = As[0];
    q.B = Bs[0];
    q.C = C;
    q.epi = epi;
    q.bias = bias;
    q.res = res;
    q.aux = aux;
    return submit_gemm(ctx, label, q);
  }
  std::vector<TileArg> T = {ta(C)};
  if (epi & TT_EPI_BIAS) T.push_back(ta(bias));
  if (epi & TT_EPI_RES) T.push_back(ta(res));
  if (epi & (TT_EPI_GELU | TT_EPI_GELU_BWD)) T.push_back(ta(aux));
  for (size_t u = 0; u < As.size(); ++u) {
    T.push_back(ta(As[u]));
    T.push_back(ta(Bs[u]));
  }
  const tt_op_gemm sc{0, tb, epi, 1.f, 0.f, 1};
  return submit_op(ctx, TT_OP_GEMM_KSUM, T.data(), (int)T.size(), &sc, sizeof(sc), label, false);
}

// whether a linear layer's contraction over several tiles runs as one K-sum
// task (else a chain of accumulating GEMM tasks), by the output tile's
// block count, the orientation of B and the contraction tile's width A0
// (measured per shape, each task alone, on the wide model's tiles):
//  * the long-K launch wins almost everywhere: 4096 x 8192 outputs (2048
//    blocks of 128x128, K 4 x 2048) 74.1 -> 67.6 ms per step for the MLP
//    input layer; 4096 x 2048 outputs (512 blocks) with 2048-wide
//    contraction tiles 1133 -> 1047 us per task (q, k, v), and with 8192-wide
//    ones and B stored [n][k] 4019 -> 3996 us (fc input gradient);
//  * except 512..1023 blocks with B stored [k][n] and contraction tiles of
//    >= 8192, where every link of the chain already runs a long K loop
//    (MLP output layer: 4062 us as a chain, 4153 us as one sum);
//  * below 512 blocks the long-K launch is split over K into slices through
//    the stream workspace (at most 128 blocks of 128 x 128: the small-tile
//    model's 1024 x 512 outputs, 32 blocks x 16 slices) or runs 64x64
//    blocks; one launch and a slice sum per task against one launch per
//    contraction tile.
// TT_KSUM_CLASSES="qkv,fc,..." forces the given task classes to K-sum tasks
// and every other class to chains (tuning).
bool use_ksum(const char* label, const TileRef& C, int tb, const TileRef& A0) {
  static std::string set;
  static int mode = -1;
  if (mode < 0) {
    const char* e = getenv("TT_KSUM_CLASSES");
    mode = e ? 1 : 0;
    if (e) set = std::string(",") + e + ",";
  }
  if (mode == 1) return set.find(std::string(",") + label + ",") != std::string::npos;
  int64_t r, c, ar, ak;
  C.t->mat(C.lin, &r, &c);
  A0.t->mat(A0.lin, &ar, &ak);
  const int64_t nb = (r / 128) * (c / 128);
  return !(nb >= 512 && nb < 1024 && !tb && ak >= 8192);
}

// whether the head's forward runs one long-K task per vocab tile (a sum over
// the embd tiles, then a separate statistics pass over the logits) instead
// of one batched launch per embd tile accumulating into the logits, the last
// one with the statistics in its epilogue. With several embd tiles the sums
// win (measured, each task alone): the wide model's head (4 embd tiles of
// 2048) 27.7 -> 25.1 ms per step (77 -> 86 % of the fp32 peak), the
// small-tile model's (16 of 512) 47.3 -> 33.9 ms, whole steps 700 -> 697 and
// 823 -> 814 ms, the statistics pass costing 0.14-0.22 ms of that. With one
// embd tile the batch and its fused statistics stay. TT_HEAD_KSUM=0/1 forces
// either (comparison).
bool head_ksum(int64_t embd_tiles) {
  static int forced = -2;
  if (forced == -2) {
    const char* e = getenv("TT_HEAD_KSUM");
    forced = e ? (atoi(e) != 0) : -1;
  }
  if (embd_tiles < 2) return false;
  return forced != 0;
}

// whether the head's last batch takes the cross-entropy statistics in its
// epilogue (else a separate pass over the logits); TT_HEAD_XSTATS=0 selects
// the separate pass (comparison)
bool head_xstats() {
  static int on = -1;
  if (on < 0) {
    const char* e = getenv("TT_HEAD_XSTATS");
    on = (e && atoi(e) == 0) ? 0 : 1;
  }
  return on == 1;
}

// tiles = value, TT_FILL_MAX_TILES tiles per task and launch (with
// pinned-host homes a task's tiles take at most an eighth of the arena)
int fill_tasks(tt_gpt2* g, const std::vector<TileRef>& tiles, float v) {
  tt_ctx* ctx = g->ctx;
  int64_t max_elems = int64_t(1) << 30;
  if (g->param_home != TT_HOME_DEVICE && ctx->budget > 0)
    max_elems = (int64_t)(ctx->budget / (8 * sizeof(float)));
  size_t k = 0;
  while (k < tiles.size()) {
    std::vector<TileRef> grp;
    int64_t elems = 0;
    while (k < tiles.size() && (int)grp.size() < TT_FILL_MAX_TILES &&
           (grp.empty() || elems + tiles[k].t->tile_elems(tiles[k].lin) <= max_elems)) {
      elems += tiles[k].t->tile_elems(tiles[k].lin);
      grp.push_back(tiles[k++]);
    }
    std::vector<TileArg> T;
    for (const TileRef& r : grp) T.push_back(ta(r));
    const tt_op_fill sc{v};
    int rc = submit_op(ctx, TT_OP_FILL, T.data(), (int)T.size(), &sc, sizeof(sc), "fill", false);
    if (rc) return rc;
  }
  return TT_OK;
}


#define TRY(x)                 \
  do {                         \
    int rc_ = (x);             \
    if (rc_ != TT_OK) return rc_; \
  } while (0)

// ------------------------------------------------------------ LayerNorm

// y = LN(x) over the embd tiles of token tile (bi, si): one task over the
// row block's feature tiles
int ln_forward(tt_gpt2* g, tt_tensor* x, tt_tensor* gam, tt_tensor* bet, tt_tensor* stats, tt_tensor* y, int64_t bi,
               int64_t si) {
  std::vector<TileArg> T;
  for (int64_t e = 0; e < g->NE; ++e) T.push_back({x, L(x, {bi, si, e})});
  for (int64_t e = 0; e < g->NE; ++e) T.push_back({gam, e});
  for (int64_t e = 0; e < g->NE; ++e) T.push_back({bet, e});
  T.push_back({stats, L(stats, {bi, si, 0})});
  for (int64_t e = 0; e < g->NE; ++e) T.push_back({y, L(y, {bi, si, e})});
  const tt_op_layernorm sc{g->c.ln_eps, 0};
  return submit_op(g->ctx, TT_OP_LAYERNORM_FWD, T.data(), (int)T.size(), &sc, sizeof(sc), "ln_fwd", false);
}

// dx (+)= LN_bwd(dy) for token tile (bi, si); dgamma/dbeta accumulate
int ln_backward(tt_gpt2* g, tt_tensor* dy, tt_tensor* x, tt_tensor* gam, tt_tensor* stats, tt_tensor* dx,
                int dx_acc, tt_tensor* dgam, tt_tensor* dbet, int64_t bi, int64_t si) {
  std::vector<TileArg> T;
  for (int64_t e = 0; e < g->NE; ++e) T.push_back({dy, L(dy, {bi, si, e})});
  for (int64_t e = 0; e < g->NE; ++e) T.push_back({x, L(x, {bi, si, e})});
  for (int64_t e = 0; e < g->NE; ++e) T.push_back({gam, e});
  T.push_back({stats, L(stats, {bi, si, 0})});
  for (int64_t e = 0; e < g->NE; ++e) T.push_back({dx, L(dx, {bi, si, e})});
  for (int64_t e = 0; e < g->NE; ++e) T.push_back({dgam, e});
  for (int64_t e = 0; e < g->NE; ++e) T.push_back({dbet, e});
  const tt_op_layernorm sc{g->c.ln_eps, dx_acc};
  return submit_op(g->ctx, TT_OP_LAYERNORM_BWD, T.data(), (int)T.size(), &sc, sizeof(sc), "ln_bwd", false);
}

// y = RMSNorm(x) over the embd tiles of token tile (bi, si): one task
int rms_forward(tt_gpt2* g, tt_tensor* x, tt_tensor* gam, tt_tensor* rstd, tt_tensor* y, int64_t bi, int64_t si) {
  std::vector<TileArg> T;
  for (int64_t e = 0; e < g->NE; ++e) T.push_back({x, L(x, {bi, si, e})});
  for (int64_t e = 0; e < g->NE; ++e) T.push_back({gam, e});
  T.push_back({rstd, L(rstd, {bi, si, 0})});
  for (int64_t e = 0; e < g->NE; ++e) T.push_back({y, L(y, {bi, si, e})});
  const tt_op_layernorm sc{g->c.ln_eps, 0};
  return submit_op(g->ctx, TT_OP_RMSNORM_FWD, T.data(), (int)T.size(), &sc, sizeof(sc), "rms_fwd", false);
}

// dx (+)= RMSNorm_bwd(dy) for token tile (bi, si); dgamma accumulates
int rms_backward(tt_gpt2* g, tt_tensor* dy, tt_tensor* x, tt_tensor* gam, tt_tensor* rstd, tt_tensor* dx,
                 int dx_acc, tt_tensor* dgam, int64_t bi, int64_t si) {
  std::vector<TileArg> T;
  for (int64_t e = 0; e < g->NE; ++e) T.push_back({dy, L(dy, {bi, si, e})});
  for (int64_t e = 0; e < g->NE; ++e) T.push_back({x, L(x, {bi, si, e})});
  for (int64_t e = 0; e < g->NE; ++e) T.push_back({gam, e});
  T.push_back({rstd, L(rstd, {bi, si, 0})});
  for (int64_t e = 0; e < g->NE; ++e) T.push_back({dx, L(dx, {bi, si, e})});
  for (int64_t e = 0; e < g->NE; ++e) T.push_back({dgam, e});
  const tt_op_layernorm sc{g->c.ln_eps, dx_acc};
  return submit_op(g->ctx, TT_OP_RMSNORM_BWD, T.data(), (int)T.size(), &sc, sizeof(sc), "rms_bwd", false);
}

// C = epi(sum_t A_t op(B_t)): one K-sum task (use_ksum) or a chain of
// accumulating GEMM tasks whose first link adds `res` and last adds `bias`
int linear(tt_ctx* ctx, const char* label, int tb, TileRef C, const std::vector<TileRef>& As,
           const std::vector<TileRef>& Bs, int epi = TT_EPI_NONE, TileRef bias = {}, TileRef res = {}) {
  if (use_ksum(label, C, tb, As[0])) return submit_ksum(ctx, label, tb, C, As, Bs, epi, bias, res);
  for (size_t t = 0; t < As.size(); ++t) {
    Gemm q;
    q.tb = tb;
    q.A = As[t];
    q.B = Bs[t];
    q.C = C;
    q.beta = t > 0 ? 1.f : 0.f;
    if (t == 0 && (epi & TT_EPI_RES)) {
      q.epi |= TT_EPI_RES;
      q.res = res;
    }
    if (t + 1 == As.size() && (epi & TT_EPI_BIAS)) {
      q.epi |= TT_EPI_BIAS;
      q.bias = bias;
    }
    if (int rc = submit_gemm(ctx, label, q)) return rc;
  }
  return TT_OK;
}

// column sums (bias gradients) of the (X, out) tile pairs: one task
int colsum_task(tt_ctx* ctx, const std::vector<TileRef>& xs, const std::vector<TileRef>& outs, int beta) {
  std::vector<TileArg> T;
  for (size_t u = 0; u < xs.size(); ++u) {
    T.push_back(ta(xs[u]));
    T.push_back(ta(outs[u]));
  }
  const tt_op_reduce sc{beta};
  return submit_op(ctx, TT_OP_REDUCE_ROWS, T.data(), (int)T.size(), &sc, sizeof(sc), "colsum", false);
}

}  // namespace

// ------------------------------------------------------------------ create

extern "C" int tt_gpt2_destroy(tt_gpt2* g) {
  if (!g) return fail(TT_ERR_ARG, "tt_gpt2_destroy: null");
  int rc = g->ctx->dryrun ? TT_OK : g->ctx->wait_all();
  if (g->graph) (void)hipGraphExecDestroy(g->graph);
  for (auto it = g->owned.rbegin(); it != g->owned.rend(); ++it) tt_tensor_destroy(*it);
  delete g;
  return rc;
}

extern "C" int tt_gpt2_set_replay(tt_gpt2* g, int on) {
  clear_error();
  if (!g) return fail(TT_ERR_ARG, "tt_gpt2_set_replay: null");
  if (on && g->ctx->dryrun) return fail(TT_ERR_UNSUPPORTED, "tt_gpt2_set_replay: dry-run context");
  // Switched off: the first GPU run of a recorded step ended in a host-side
  // segmentation fault whose cause has not been found; the recording path
  // stays unreachable until it is.
  if (on) return fail(TT_ERR_UNSUPPORTED, "tt_gpt2_set_replay: graph replay is disabled in this build");
  if (on && g->param_home != TT_HOME_DEVICE)
    return fail(TT_ERR_UNSUPPORTED, "tt_gpt2_set_replay: pinned-host parameters are staged at launch time");
  if (!on && g->graph) {
    TRY(g->ctx->wait_all());
    (void)hipGraphExecDestroy(g->graph);
    g->graph = nullptr;
  }
  g->replay = on != 0;
  return TT_OK;
}

static int create_model(tt_ctx* ctx, const tt_gpt2_config* cfg, const tt_gpt2_tiles* tiles, int param_home,
                        bool llama, tt_gpt2** out) {
  clear_error();
  if (!ctx || !cfg || !tiles || !out) return fail(TT_ERR_ARG, "tt_gpt2_create: null argument");
  const tt_gpt2_config& c = *cfg;
  const tt_gpt2_tiles& t = *tiles;
  if (c.n_layer < 0 || c.vocab < 1 || c.n_embd < 1 || c.n_head < 1 || c.n_inner < 1 || c.seq < 1 || c.batch < 1)
    return fail(TT_ERR_ARG, "tt_gpt2_create: sizes must be positive");
  if (t.batch < 1 || t.seq < 1 || t.embd < 1 || t.inner < 1 || t.head < 1 || t.vocab < 1)
    return fail(TT_ERR_ARG, "tt_gpt2_create: tiles must be positive");
  if (c.n_embd % c.n_head) return fail(TT_ERR_SHAPE, "tt_gpt2_create: n_embd %% n_head != 0");
  if (c.seq % t.seq) return fail(TT_ERR_SHAPE, "tt_gpt2_create: seq tile must divide seq");
  if (c.n_head % t.head) return fail(TT_ERR_SHAPE, "tt_gpt2_create: head tile must divide n_head");
  if (c.batch % t.batch) return fail(TT_ERR_SHAPE, "tt_gpt2_create: batch tile must divide batch");
  const int64_t hd = c.n_embd / c.n_head;
  if (hd != 16 && hd != 32 && hd != 64 && hd != 128)
    return fail(TT_ERR_UNSUPPORTED, "tt_gpt2_create: head dim %lld not in {16,32,64,128}", (long long)hd);
  const int64_t et = std::min(t.embd, c.n_embd), vt = std::min(t.vocab, c.vocab);
  if (et > 2048 || vt > 2048) return fail(TT_ERR_UNSUPPORTED, "tt_gpt2_create: embd and vocab tiles must be <= 2048");
  if (param_home != TT_HOME_DEVICE && param_home != TT_HOME_PINNED_HOST && param_home != TT_HOME_PINNED_STATE)
    return fail(TT_ERR_ARG, "tt_gpt2_create: bad param_home");
  // the RMSNorm kernels take float4 rows of at most 16384 features
  if (llama && (c.n_embd % 4 || et % 4 || c.n_embd > 16384))
    return fail(TT_ERR_SHAPE, "tt_llama_create: n_embd and the embd tile must be multiples of 4, n_embd <= 16384");

  std::unique_ptr<tt_gpt2> g(new tt_gpt2());
  g->ctx = ctx;
  g->c = c;
  g->t = t;
  g->param_home = param_home;
  g->llama = llama;
  g->nb = c.batch / t.batch;
  g->ns = c.seq / t.seq;
  g->ntok = g->nb * g->ns;
  g->rows = (int64_t)t.batch * t.seq;
  g->NE = ceil_div(c.n_embd, et);
  g->NI = ceil_div(c.n_inner, std::min(t.inner, c.n_inner));
  g->NH = c.n_head / t.head;
  g->NV = ceil_div(c.vocab, vt);
  g->hd = hd;
  const int64_t B = c.batch, T = c.seq, d = c.n_embd, H = c.n_head, I = c.n_inner, V = c.vocab;
  const int64_t bt = t.batch, sq = t.seq, it = t.inner, ht = t.head;
  const int ph = param_home;
  tt_gpt2* G = g.get();
  auto fail_clean = [&](int rc) {
    for (auto p = G->owned.rbegin(); p != G->owned.rend(); ++p) tt_tensor_destroy(*p);
    G->owned.clear();
    return rc;
  };
#define MK(...)                          \
  do {                                   \
    int rc_ = mk(G, __VA_ARGS__);        \
    if (rc_) return fail_clean(rc_);     \
  } while (0)
  // parameters, gradients and moments in param_specs order
  struct Spec {
    const char* name;
    std::vector<int64_t> shape, tile;
    int split;
  };
  std::vector<Spec> specs;
  specs.push_back({"wte", {V, d}, {vt, et}, 1});
  if (llama) {
    for (int l = 0; l < c.n_layer; ++l) {
      specs.push_back({"attn_norm_g", {d}, {et}, 0});
      specs.push_back({"w_qkv", {d, 3, H, hd}, {et, 1, ht, hd}, 1});
      specs.push_back({"w_o", {H, hd, d}, {ht, hd, et}, 2});
      specs.push_back({"mlp_norm_g", {d}, {et}, 0});
      specs.push_back({"w_gate", {d, I}, {et, it}, 1});
      specs.push_back({"w_up", {d, I}, {et, it}, 1});
      specs.push_back({"w_down", {I, d}, {it, et}, 1});
    }
    specs.push_back({"norm_f_g", {d}, {et}, 0});
    specs.push_back({"w_head", {V, d}, {vt, et}, 1});
  } else {
  specs.push_back({"wpe", {T, d}, {sq, et}, 1});
  for (int l = 0; l < c.n_layer; ++l) {
    specs.push_back({"ln1_g", {d}, {et}, 0});
    specs.push_back({"ln1_b", {d}, {et}, 0});
    specs.push_back({"w_qkv", {d, 3, H, hd}, {et, 1, ht, hd}, 1});
    specs.push_back({"b_qkv", {3, H, hd}, {1, ht, hd}, 0});
    specs.push_back({"w_o", {H, hd, d}, {ht, hd, et}, 2});
    specs.push_back({"b_o", {d}, {et}, 0});
    specs.push_back({"ln2_g", {d}, {et}, 0});
    specs.push_back({"ln2_b", {d}, {et}, 0});
    specs.push_back({"w_fc", {d, I}, {et, it}, 1});
    specs.push_back({"b_fc", {I}, {it}, 0});
    specs.push_back({"w_p", {I, d}, {it, et}, 1});
    specs.push_back({"b_p", {d}, {et}, 0});
  }
  specs.push_back({"lnf_g", {d}, {et}, 0});
  specs.push_back({"lnf_b", {d}, {et}, 0});
  }
  for (auto& s : specs) {
    tt_tensor* ts[4];
    const char* suffix[4] = {"", ".grad", ".m", ".v"};
    for (int j = 0; j < 4; ++j) {
      std::string nm = std::string(s.name) + suffix[j];
      // TT_HOME_PINNED_STATE: parameters and moments pinned, gradients in HBM
      const int home = ph == TT_HOME_DEVICE ? TT_HOME_DEVICE
                       : (ph == TT_HOME_PINNED_STATE && j == 1) ? TT_HOME_DEVICE
                                                                 : TT_HOME_PINNED_HOST;
      int rc = tensor_create(ctx, (int)s.shape.size(), s.shape.data(), s.tile.data(), TT_F32, home, s.split,
                             nm.c_str(), &ts[j]);
      if (rc) return fail_clean(rc);
      G->owned.push_back(ts[j]);
    }
    G->P.push_back(ts[0]);
    G->G.push_back(ts[1]);
    G->M.push_back(ts[2]);
    G->Vv.push_back(ts[3]);
  }
  // tokens and per-token-tile index tensors
  MK(&G->tokens, "tokens", {B, T + 1}, {B, T + 1}, 1, TT_I32);
  MK(&G->ids, "ids", {B, T}, {bt, sq}, 2, TT_I32);
  MK(&G->labels, "labels", {B, T}, {bt, sq}, 2, TT_I32);
  MK(&G->sorted, "sorted_ids", {B, T}, {bt, sq}, 2, TT_I32);
  MK(&G->perm, "perm", {B, T}, {bt, sq}, 2, TT_I32);
  // activations
  G->blk.resize(c.n_layer);
  MK(&(G->blk.empty() ? G->h_last : G->blk[0].h_in), "h0", {B, T, d}, {bt, sq, et}, 2);
  const int64_t nstat = llama ? 1 : 2;  // (mean, rstd) or rstd per row
  for (int l = 0; l < c.n_layer; ++l) {
    BlockT& b = G->blk[l];
    MK(&b.ln1, "ln1_stats", {B, T, nstat}, {bt, sq, nstat}, 2);
    MK(&b.n1, "n1", {B, T, d}, {bt, sq, et}, 2);
    MK(&b.q, "q", {B, T, H, hd}, {bt, sq, ht, hd}, 2);
    MK(&b.k, "k", {B, T, H, hd}, {bt, sq, ht, hd}, 2);
    MK(&b.v, "v", {B, T, H, hd}, {bt, sq, ht, hd}, 2);
    MK(&b.o, "o", {B, T, H, hd}, {bt, sq, ht, hd}, 2);
    MK(&b.lse, "attn_lse", {B / bt, T / sq, H / ht, bt * sq * ht}, {1, 1, 1, bt * sq * ht}, 3);
    MK(&b.h_mid, "h_mid", {B, T, d}, {bt, sq, et}, 2);
    MK(&b.ln2, "ln2_stats", {B, T, nstat}, {bt, sq, nstat}, 2);
    MK(&b.n2, "n2", {B, T, d}, {bt, sq, et}, 2);
    MK(&b.u, "u", {B, T, I}, {bt, sq, it}, 2);
    MK(&b.g, llama ? "swiglu" : "gelu", {B, T, I}, {bt, sq, it}, 2);
    if (llama) MK(&b.a, "gate", {B, T, I}, {bt, sq, it}, 2);
    tt_tensor** next = (l + 1 < c.n_layer) ? &G->blk[l + 1].h_in : &G->h_last;
    MK(next, "h", {B, T, d}, {bt, sq, et}, 2);
  }
  MK(&G->lnf, "lnf_stats", {B, T, nstat}, {bt, sq, nstat}, 2);
  if (llama) MK(&G->rope, "rope_table", {T, hd}, {T, hd}, 1);
  MK(&G->nf, "nf", {B, T, d}, {bt, sq, et}, 2);
  MK(&G->z, "logits", {B, T, V}, {bt, sq, vt}, 2);
  MK(&G->ml, "attn_ml", {B / bt, T / sq, H / ht, bt * sq * ht * 2}, {1, 1, 1, bt * sq * ht * 2}, 3);
  // cross-entropy partials per (vocab tile, token tile): one (max, sum exp,
  // picked) triple per row for each 64-column group of the vocab tile (the
  // head's statistics epilogue), or one per tile (the separate statistics pass)
  const int64_t xgroups = (vt + 63) / 64;
  MK(&G->ce_parts, "ce_parts", {G->NV, G->ntok, xgroups * G->rows * 3}, {1, 1, xgroups * G->rows * 3}, 2);
  MK(&G->ce_lse, "ce_lse", {G->ntok, G->rows}, {1, G->rows}, 1);
  MK(&G->row_loss, "row_loss", {G->ntok, G->rows}, {1, G->rows}, 1);
  MK(&G->loss, "loss", {1}, {1}, 0);
  MK(&G->dnf, "dnf", {B, T, d}, {bt, sq, et}, 2);
  MK(&G->dh, "dh", {B, T, d}, {bt, sq, et}, 2);
  MK(&G->dgu, "dgu", {B, T, I}, {bt, sq, it}, 2);
  MK(&G->dn, "dn", {B, T, d}, {bt, sq, et}, 2);
  MK(&G->dO, "do", {B, T, H, hd}, {bt, sq, ht, hd}, 2);
  MK(&G->dq, "dq", {B, T, H, hd}, {bt, sq, ht, hd}, 2);
  MK(&G->dk, "dk", {B, T, H, hd}, {bt, sq, ht, hd}, 2);
  MK(&G->dv, "dv", {B, T, H, hd}, {bt, sq, ht, hd}, 2);
  MK(&G->Dv, "attn_D", {B / bt, T / sq, H / ht, bt * sq * ht}, {1, 1, 1, bt * sq * ht}, 3);
  MK(&G->step, "adam_step", {1}, {1}, 0, TT_I32);
  MK(&G->bc, "adam_bias_corr", {2}, {2}, 0);
#undef MK
  // per-stream workspace: LayerNorm partial statistics and column sums, the
  // deterministic column sums of the bias gradients (up to 16 tiles per
  // task), split-K partial sums
  const int64_t widest = std::max<int64_t>({et, std::min<int64_t>(it, I), ht * hd});
  size_t ws = std::max(layernorm_fwd_workspace(G->NE, G->rows), layernorm_bwd_workspace(G->NE, G->rows, et));
  ws = std::max(ws, std::min<int64_t>(16, std::max(G->NE, G->NI)) * tile_reduce_rows_workspace(G->rows, widest));
  // the q/k/v bias gradients: up to 15 head tiles per multi-tile column sum
  ws = std::max(ws, tile_reduce_rows_workspace(G->rows, std::min<int64_t>(15, 3 * G->NH) * ht * hd));
  if (llama) ws = std::max(ws, tile_rmsnorm_bwd_workspace(G->rows, d));
  // dS of one attention tile pair (the backward's dK/dV kernel hands it to the dQ kernel)
  ws = std::max(ws, tile_attention_bwd_workspace(bt, ht, sq, sq));
  // K slices of the linear layers' long-K sums over token-tile outputs
  for (int64_t cols : {et, std::min<int64_t>(it, I), ht * hd, vt})
    ws = std::max(ws, tile_gemm_ksum_workspace(G->rows, cols));
  {
    // split-K slices of the step's GEMM shapes (m, n, k), capped at 256 MiB per stream
    const int64_t r = G->rows, e = et, in = std::min<int64_t>(it, I), hw = ht * hd, vv = vt;
    const int64_t shapes[][3] = {{r, hw, e}, {r, e, hw}, {r, in, e}, {r, e, in}, {r, vv, e}, {vv, e, r}, {r, e, vv},
                                 {in, e, r}, {e, in, r}, {hw, e, r}, {e, hw, r}};
    size_t g = 0;
    for (auto& s : shapes) g = std::max(g, tile_gemm_workspace(s[0], s[1], s[2]));
    {  // the batched weight gradients of one token tile (q/k/v, attention
       // projection, fc, MLP projection), split-K when the products are few
      auto batch = [&](int64_t cnt, int64_t m, int64_t n) {
        std::vector<int64_t> bm(cnt, m), bn(cnt, n);
        g = std::max(g, tile_gemm_batch_workspace((int)cnt, bm.data(), bn.data(), r));
      };
      batch(3 * G->NH * G->NE, e, hw);
      batch(G->NE * G->NH, hw, e);
      batch(G->NI * G->NE * (llama ? 2 : 1), e, in);  // LLaMA: gate and up weights in one batch
      batch(G->NE * G->NI, in, e);
    }
    ws = std::max(ws, std::min<size_t>(g, (size_t)256 << 20));
  }
  if (int rc = ctx->ensure_workspace(ws)) return fail_clean(rc);
  // zero gradients' home state, moments and the step counter
  if (!ctx->dryrun) {
    for (size_t i = 0; i < G->P.size(); ++i)
      for (tt_tensor* x : {G->M[i], G->Vv[i]})
        if (x->home == TT_HOME_DEVICE) {
          hipError_t e = hipMemset(x->base, 0, x->bytes());
          if (e != hipSuccess) return fail_clean(fail(TT_ERR_HIP, "hipMemset: %s", hipGetErrorString(e)));
        }
    if (hipMemset(G->step->base, 0, 4) != hipSuccess) return fail_clean(fail(TT_ERR_HIP, "hipMemset(step)"));
  }
  if (llama) {  // the rotary table, once (every rope task reads it)
    const TileArg T1[1] = {{G->rope, 0}};
    const tt_op_rope sc{0, 0, 10000.0};
    if (int rc = submit_op(ctx, TT_OP_ROPE_TABLE, T1, 1, &sc, sizeof(sc), "rope_table", false)) return fail_clean(rc);
  }
  *out = g.release();
  return TT_OK;
}

extern "C" int tt_gpt2_create(tt_ctx* ctx, const tt_gpt2_config* cfg, const tt_gpt2_tiles* tiles, int param_home,
                              tt_gpt2** out) {
  return create_model(ctx, cfg, tiles, param_home, false, out);
}

extern "C" int tt_llama_create(tt_ctx* ctx, const tt_gpt2_config* cfg, const tt_gpt2_tiles* tiles, int param_home,
                               tt_gpt2** out) {
  return create_model(ctx, cfg, tiles, param_home, true, out);
}

extern "C" int tt_gpt2_num_params(tt_gpt2* g, int* n) {
  if (!g || !n) return fail(TT_ERR_ARG, "tt_gpt2_num_params: null");
  *n = (int)g->P.size();
  return TT_OK;
}

extern "C" int tt_gpt2_param(tt_gpt2* g, int index, tt_tensor** p, tt_tensor** gr, tt_tensor** m, tt_tensor** v) {
  if (!g) return fail(TT_ERR_ARG, "tt_gpt2_param: null");
  if (index < 0 || index >= (int)g->P.size()) return fail(TT_ERR_ARG, "tt_gpt2_param: index %d out of range", index);
  if (p) *p = g->P[index];
  if (gr) *gr = g->G[index];
  if (m) *m = g->M[index];
  if (v) *v = g->Vv[index];
  return TT_OK;
}

extern "C" int tt_gpt2_task_count(tt_gpt2* g, int64_t* n) {
  if (!g || !n) return fail(TT_ERR_ARG, "tt_gpt2_task_count: null");
  *n = g->last_tasks;
  return TT_OK;
}

extern "C" int tt_gpt2_loss(tt_gpt2* g, float* loss) {
  clear_error();
  if (!g || !loss) return fail(TT_ERR_ARG, "tt_gpt2_loss: null");
  if (g->ctx->dryrun) {
    *loss = NAN;
    return g->ctx->wait_all();
  }
  TRY(g->ctx->wait_all());
  TT_HIP_TRY(hipMemcpy(loss, g->loss->base, 4, hipMemcpyDeviceToHost));
  return TT_OK;
}

extern "C" int tt_gpt2_row_losses(tt_gpt2* g, float* out) {
  clear_error();
  if (!g || !out) return fail(TT_ERR_ARG, "tt_gpt2_row_losses: null");
  if (g->ctx->dryrun) return fail(TT_ERR_STATE, "tt_gpt2_row_losses: dry-run context");
  // row_loss is [token tile, row]: token tile bi + nb*si holds rows (b in the
  // batch tile) * seq_tile + (t in the seq tile)
  std::vector<float> tiles((size_t)(g->ntok * g->rows));
  TRY(tt_tensor_copy_out(g->row_loss, tiles.data()));
  const int64_t T = g->c.seq, bt = g->t.batch, sq = g->t.seq;
  for (int64_t b = 0; b < g->c.batch; ++b)
    for (int64_t t = 0; t < T; ++t) {
      const int64_t ti = b / bt + g->nb * (t / sq), r = (b % bt) * sq + t % sq;
      out[b * T + t] = tiles[ti * g->rows + r];
    }
  return TT_OK;
}

// -------------------------------------------------------------------- step

static int submit_step(tt_gpt2* g, const int32_t* tokens, const tt_adamw_hparams* hp, int do_update, int micro,
                       int n_micro);

// learning rate of AdamW iteration t (from 1): start_lr at 1, lr from
// full_lr_iter on, linear in between (the README's warm-up flags)
static_assert(TT_SGD_MAX_TILES >= TT_ADAMW_MAX_TILES, "SGD groups are formed with the AdamW group size");

static float lr_at(int64_t t, const tt_adamw_hparams& h) {
  if (h.full_lr_iter <= 1 || t >= h.full_lr_iter) return h.lr;
  return h.start_lr + (h.lr - h.start_lr) * (float)(t - 1) / (float)(h.full_lr_iter - 1);
}

// every minibatch's tasks; `h` carries the lr of this update
static int submit_batch(tt_gpt2* g, const int32_t* tokens, int n_micro, const tt_adamw_hparams& h, int do_update) {
  tt_ctx* ctx = g->ctx;
  const int64_t t0 = ctx->next_id, win = (int64_t)g->c.batch * (g->c.seq + 1);
  for (int i = 0; i < n_micro; ++i)
    TRY(submit_step(g, tokens ? tokens + i * win : nullptr, &h, do_update && i == n_micro - 1, i, n_micro));
  g->last_tasks = ctx->next_id - t0;
  return TT_OK;
}

extern "C" int tt_gpt2_step_accum(tt_gpt2* g, const int32_t* tokens, int n_micro, const tt_adamw_hparams* hp,
                                  int do_update) {
  clear_error();
  if (!g || !hp) return fail(TT_ERR_ARG, "tt_gpt2_step: null argument");
  if (n_micro < 1) return fail(TT_ERR_ARG, "tt_gpt2_step_accum: n_micro must be >= 1");
  if (hp->optimizer != TT_OPT_ADAMW && hp->optimizer != TT_OPT_SGD)
    return fail(TT_ERR_ARG, "tt_gpt2_step: unknown optimizer");
  tt_ctx* ctx = g->ctx;
  if (!tokens && !ctx->dryrun) return fail(TT_ERR_ARG, "tt_gpt2_step: null tokens");
  tt_adamw_hparams h = *hp;
  if (do_update) h.lr = lr_at(g->updates + 1, *hp);
  if (!g->replay || n_micro != 1) {
    TRY(submit_batch(g, tokens, n_micro, h, do_update));
    if (do_update) g->updates++;
    return TT_OK;
  }
  const bool same = g->graph && g->graph_tokens == tokens && g->graph_update == do_update &&
                    !memcmp(&g->graph_hp, &h, sizeof(h)) && g->graph_ws_gen == ctx->workspace_gen;
  if (!same) {
    if (g->graph) {
      TRY(ctx->wait_all());
      (void)hipGraphExecDestroy(g->graph);
      g->graph = nullptr;
    }
    TRY(ctx->capture_begin());
    const int rc = submit_batch(g, tokens, 1, h, do_update);
    hipGraphExec_t exec = nullptr;
    const int rc2 = ctx->capture_end(rc == TT_OK ? &exec : nullptr);
    if (rc != TT_OK) return rc;
    if (rc2 != TT_OK) return rc2;
    g->graph = exec;
    g->graph_tokens = tokens;
    g->graph_hp = h;
    g->graph_update = do_update;
    g->graph_tasks = g->last_tasks;
    g->graph_ws_gen = ctx->workspace_gen;
  }
  g->last_tasks = g->graph_tasks;
  TRY(ctx->graph_launch(g->graph));
  if (do_update) g->updates++;
  return TT_OK;
}

extern "C" int tt_gpt2_step(tt_gpt2* g, const int32_t* tokens, const tt_adamw_hparams* hp, int do_update) {
  return tt_gpt2_step_accum(g, tokens, 1, hp, do_update);
}

// Causal attention of one block: (query tile, key tile) pairs, key tiles in order
static int attention_forward(tt_gpt2* g, BlockT& b) {
  tt_ctx* ctx = g->ctx;
  const int64_t sq = g->t.seq;
  const float scale = 1.f / std::sqrt((float)g->hd);
  for (int64_t bi = 0; bi < g->nb; ++bi)
    for (int64_t hj = 0; hj < g->NH; ++hj)
      for (int64_t qi = 0; qi < g->ns; ++qi)
        for (int64_t ki = 0; ki <= qi; ++ki) {
          const int64_t lq = L(b.q, {bi, qi, hj, 0}), lk = L(b.k, {bi, ki, hj, 0});
          const TileArg T[6] = {{b.q, lq}, {b.k, lk}, {b.v, lk}, {b.o, lq}, {g->ml, L(g->ml, {bi, qi, hj, 0})},
                                {b.lse, L(b.lse, {bi, qi, hj, 0})}};
          const tt_op_attention sc{qi * sq, ki * sq, ki == 0, ki == qi, 0, 0, scale};
          TRY(submit_op(ctx, TT_OP_ATTENTION_FWD, T, 6, &sc, sizeof(sc), "attn_fwd", false));
        }
  return TT_OK;
}

// its backward: D = rowsum(dO * O) per query tile, then dQ, dK, dV over the
// tile pairs (dK, dV accumulating over query tiles, dQ over key tiles)
static int attention_backward(tt_gpt2* g, BlockT& b) {
  tt_ctx* ctx = g->ctx;
  const int64_t sq = g->t.seq;
  const float scale = 1.f / std::sqrt((float)g->hd);
  for (int64_t bi = 0; bi < g->nb; ++bi)
    for (int64_t hj = 0; hj < g->NH; ++hj) {
      for (int64_t qi = 0; qi < g->ns; ++qi) {
        const int64_t lq = L(b.o, {bi, qi, hj, 0});
        const TileArg T[3] = {{b.o, lq}, {g->dO, lq}, {g->Dv, L(g->Dv, {bi, qi, hj, 0})}};
        const tt_op_attention sc{0, 0, 0, 0, 0, 0, scale};
        TRY(submit_op(ctx, TT_OP_ATTENTION_PREP, T, 3, &sc, sizeof(sc), "attn_prep", false));
      }
      for (int64_t qi = 0; qi < g->ns; ++qi)
        for (int64_t ki = 0; ki <= qi; ++ki) {
          const int64_t lq = L(b.q, {bi, qi, hj, 0}), lk = L(b.k, {bi, ki, hj, 0});
          const int64_t ls = L(b.lse, {bi, qi, hj, 0});
          const TileArg T[9] = {{b.q, lq},   {b.k, lk},   {b.v, lk},   {g->dO, lq}, {b.lse, ls},
                                {g->Dv, ls}, {g->dq, lq}, {g->dk, lk}, {g->dv, lk}};
          const tt_op_attention sc{qi * sq, ki * sq, 0, 0, ki > 0, qi > ki, scale};
          TRY(submit_op(ctx, TT_OP_ATTENTION_BWD, T, 9, &sc, sizeof(sc), "attn_bwd", false));
        }
    }
  return TT_OK;
}

// the rotary embedding of every head tile's q and k (or, inverse, of dq and
// dk) for token tile (bi, si), in place: one task per head tile
static int rope_tasks(tt_gpt2* g, tt_tensor* q, tt_tensor* k, int64_t bi, int64_t si, int inverse) {
  for (int64_t hj = 0; hj < g->NH; ++hj) {
    const int64_t lq = L(q, {bi, si, hj, 0});
    const TileArg T[3] = {{q, lq}, {k, lq}, {g->rope, 0}};
    const tt_op_rope sc{si * g->t.seq, inverse, 10000.0};
    TRY(submit_op(g->ctx, TT_OP_ROPE, T, 3, &sc, sizeof(sc), inverse ? "rope_bwd" : "rope", false));
  }
  return TT_OK;
}

// h_out = h_mid + silu(n2 W_gate) * (n2 W_up) W_down over the token tile's
// inner tiles, up to 16 (gate, up, out) triples per SwiGLU task
static int swiglu_tasks(tt_gpt2* g, BlockT& b, tt_tensor* first, int64_t bi, int64_t si, bool bwd) {
  for (int64_t i0 = 0; i0 < g->NI; i0 += 16) {
    std::vector<TileArg> T;
    for (int64_t ij = i0; ij < std::min(g->NI, i0 + 16); ++ij) {
      if (bwd) {  // (dh, a, u): a and u replaced by their gradients
        T.push_back({first, L(first, {bi, si, ij})});
        T.push_back({b.a, L(b.a, {bi, si, ij})});
        T.push_back({b.u, L(b.u, {bi, si, ij})});
      } else {    // (a, u, g)
        T.push_back({b.a, L(b.a, {bi, si, ij})});
        T.push_back({b.u, L(b.u, {bi, si, ij})});
        T.push_back({b.g, L(b.g, {bi, si, ij})});
      }
    }
    TRY(submit_op(g->ctx, bwd ? TT_OP_SWIGLU_BWD : TT_OP_SWIGLU_FWD, T.data(), (int)T.size(), nullptr, 0,
                  bwd ? "swiglu_bwd" : "swiglu", false));
  }
  return TT_OK;
}

// One LLaMA block forward: h_mid = h_in + Attn(rope(RMS1(h_in) W_q), rope(.. W_k), .. W_v) W_o,
// h_out = h_mid + SwiGLU(RMS2(h_mid)) W_down
static int llama_block_forward(tt_gpt2* g, int l) {
  tt_ctx* ctx = g->ctx;
  BlockT& b = g->blk[l];
  tt_tensor* hout = (l + 1 < g->c.n_layer) ? g->blk[l + 1].h_in : g->h_last;
  tt_tensor *an = g->P[g->lidx(l, ANORM)], *wqkv = g->P[g->lidx(l, LQKV)], *wo = g->P[g->lidx(l, LWO)];
  tt_tensor *mn = g->P[g->lidx(l, MNORM)], *wg = g->P[g->lidx(l, LGATE)], *wu = g->P[g->lidx(l, LUP)];
  tt_tensor* wd = g->P[g->lidx(l, LDOWN)];
  const int64_t NE = g->NE, NI = g->NI, NH = g->NH;
  tt_tensor* qkv[3] = {b.q, b.k, b.v};
  for (int64_t bi = 0; bi < g->nb; ++bi)
    for (int64_t si = 0; si < g->ns; ++si) {
      TRY(rms_forward(g, b.h_in, an, b.ln1, b.n1, bi, si));
      for (int cq = 0; cq < 3; ++cq)
        for (int64_t hj = 0; hj < NH; ++hj) {
          std::vector<TileRef> As, Bs;
          for (int64_t ek = 0; ek < NE; ++ek) {
            As.push_back({b.n1, L(b.n1, {bi, si, ek})});
            Bs.push_back({wqkv, L(wqkv, {ek, cq, hj, 0})});
          }
          TRY(linear(ctx, "qkv", 0, {qkv[cq], L(qkv[cq], {bi, si, hj, 0})}, As, Bs));
        }
      TRY(rope_tasks(g, b.q, b.k, bi, si, 0));
    }
  TRY(attention_forward(g, b));
  for (int64_t bi = 0; bi < g->nb; ++bi)
    for (int64_t si = 0; si < g->ns; ++si) {
      for (int64_t ej = 0; ej < NE; ++ej) {
        std::vector<TileRef> As, Bs;
        for (int64_t hk = 0; hk < NH; ++hk) {
          As.push_back({b.o, L(b.o, {bi, si, hk, 0})});
          Bs.push_back({wo, L(wo, {hk, 0, ej})});
        }
        TRY(linear(ctx, "attn_proj", 0, {b.h_mid, L(b.h_mid, {bi, si, ej})}, As, Bs, TT_EPI_RES, {},
                   {b.h_in, L(b.h_in, {bi, si, ej})}));
      }
      TRY(rms_forward(g, b.h_mid, mn, b.ln2, b.n2, bi, si));
      for (int64_t ij = 0; ij < NI; ++ij)
        for (tt_tensor* w : {wg, wu}) {
          std::vector<TileRef> As, Bs;
          for (int64_t ek = 0; ek < NE; ++ek) {
            As.push_back({b.n2, L(b.n2, {bi, si, ek})});
            Bs.push_back({w, L(w, {ek, ij})});
          }
          tt_tensor* out = w == wg ? b.a : b.u;
          TRY(linear(ctx, "fc", 0, {out, L(out, {bi, si, ij})}, As, Bs));
        }
      TRY(swiglu_tasks(g, b, nullptr, bi, si, false));
      for (int64_t ej = 0; ej < NE; ++ej) {
        std::vector<TileRef> As, Bs;
        for (int64_t ik = 0; ik < NI; ++ik) {
          As.push_back({b.g, L(b.g, {bi, si, ik})});
          Bs.push_back({wd, L(wd, {ik, ej})});
        }
        TRY(linear(ctx, "mlp_proj", 0, {hout, L(hout, {bi, si, ej})}, As, Bs, TT_EPI_RES, {},
                   {b.h_mid, L(b.h_mid, {bi, si, ej})}));
      }
    }
  return TT_OK;
}

// Its backward; g->dh holds dL/dh_out on entry and dL/dh_in on return, and
// the block's weight gradients are written (first token tile of the first
// minibatch) or accumulated
static int llama_block_backward(tt_gpt2* g, int l, bool later_mb) {
  tt_ctx* ctx = g->ctx;
  BlockT& b = g->blk[l];
  tt_tensor *an = g->P[g->lidx(l, ANORM)], *wqkv = g->P[g->lidx(l, LQKV)], *wo = g->P[g->lidx(l, LWO)];
  tt_tensor *mn = g->P[g->lidx(l, MNORM)], *wg = g->P[g->lidx(l, LGATE)], *wu = g->P[g->lidx(l, LUP)];
  tt_tensor* wd = g->P[g->lidx(l, LDOWN)];
  tt_tensor *gwqkv = g->G[g->lidx(l, LQKV)], *gwo = g->G[g->lidx(l, LWO)], *gwg = g->G[g->lidx(l, LGATE)];
  tt_tensor *gwu = g->G[g->lidx(l, LUP)], *gwd = g->G[g->lidx(l, LDOWN)];
  const int64_t NE = g->NE, NI = g->NI, NH = g->NH;
  tt_tensor* dqkv[3] = {g->dq, g->dk, g->dv};
  for (int64_t si = 0; si < g->ns; ++si)
    for (int64_t bi = 0; bi < g->nb; ++bi) {
      const int64_t ti = bi + g->nb * si;
      const float wbeta = (ti > 0 || later_mb) ? 1.f : 0.f;
      // MLP: h_out = h_mid + g W_down, g = silu(a) * u
      {
        std::vector<Gemm> qs;
        for (int64_t ej = 0; ej < NE; ++ej)
          for (int64_t ik = 0; ik < NI; ++ik) {
            Gemm q;
            q.ta = 1;
            q.A = {b.g, L(b.g, {bi, si, ik})};
            q.B = {g->dh, L(g->dh, {bi, si, ej})};
            q.C = {gwd, L(gwd, {ik, ej})};
            q.beta = wbeta;
            qs.push_back(q);
          }
        TRY(submit_gemm_batch(ctx, "mlp_proj_dw", qs, true));
      }
      for (int64_t ik = 0; ik < NI; ++ik) {
        std::vector<TileRef> As, Bs;
        for (int64_t ej = 0; ej < NE; ++ej) {
          As.push_back({g->dh, L(g->dh, {bi, si, ej})});
          Bs.push_back({wd, L(wd, {ik, ej})});
        }
        TRY(linear(ctx, "mlp_proj_dx", 1, {g->dgu, L(g->dgu, {bi, si, ik})}, As, Bs));
      }
      TRY(swiglu_tasks(g, b, g->dgu, bi, si, true));  // a <- da, u <- du
      {
        std::vector<Gemm> qs;
        for (int64_t ik = 0; ik < NI; ++ik)
          for (int64_t ek = 0; ek < NE; ++ek)
            for (int w = 0; w < 2; ++w) {
              tt_tensor *src = w ? b.u : b.a, *dst = w ? gwu : gwg;
              Gemm q;
              q.ta = 1;
              q.A = {b.n2, L(b.n2, {bi, si, ek})};
              q.B = {src, L(src, {bi, si, ik})};
              q.C = {dst, L(dst, {ek, ik})};
              q.beta = wbeta;
              qs.push_back(q);
            }
        TRY(submit_gemm_batch(ctx, "fc_dw", qs, true));
      }
      // dn2 = da W_gate^T + du W_up^T: one sum over both weights' inner tiles
      for (int64_t ek = 0; ek < NE; ++ek) {
        std::vector<TileRef> As, Bs;
        for (int w = 0; w < 2; ++w)
          for (int64_t ik = 0; ik < NI; ++ik) {
            tt_tensor *src = w ? b.u : b.a, *wt = w ? wu : wg;
            As.push_back({src, L(src, {bi, si, ik})});
            Bs.push_back({wt, L(wt, {ek, ik})});
          }
        TRY(linear(ctx, "fc_dx", 1, {g->dn, L(g->dn, {bi, si, ek})}, As, Bs));
      }
      TRY(rms_backward(g, g->dn, b.h_mid, mn, b.ln2, g->dh, 1, g->G[g->lidx(l, MNORM)], bi, si));
      // attention projection: h_mid = h_in + O W_o
      {
        std::vector<Gemm> qs;
        for (int64_t ej = 0; ej < NE; ++ej)
          for (int64_t hk = 0; hk < NH; ++hk) {
            Gemm q;
            q.ta = 1;
            q.A = {b.o, L(b.o, {bi, si, hk, 0})};
            q.B = {g->dh, L(g->dh, {bi, si, ej})};
            q.C = {gwo, L(gwo, {hk, 0, ej})};
            q.beta = wbeta;
            qs.push_back(q);
          }
        TRY(submit_gemm_batch(ctx, "attn_proj_dw", qs, true));
      }
      for (int64_t hk = 0; hk < NH; ++hk) {
        std::vector<TileRef> As, Bs;
        for (int64_t ej = 0; ej < NE; ++ej) {
          As.push_back({g->dh, L(g->dh, {bi, si, ej})});
          Bs.push_back({wo, L(wo, {hk, 0, ej})});
        }
        TRY(linear(ctx, "attn_proj_dx", 1, {g->dO, L(g->dO, {bi, si, hk, 0})}, As, Bs));
      }
    }
  TRY(attention_backward(g, b));
  for (int64_t si = 0; si < g->ns; ++si)
    for (int64_t bi = 0; bi < g->nb; ++bi) {
      const int64_t ti = bi + g->nb * si;
      // gradients of the rotated q and k back through the rotation
      TRY(rope_tasks(g, g->dq, g->dk, bi, si, 1));
      std::vector<Gemm> qs;
      for (int cq = 0; cq < 3; ++cq)
        for (int64_t hj = 0; hj < NH; ++hj)
          for (int64_t ek = 0; ek < NE; ++ek) {
            Gemm q;
            q.ta = 1;
            q.A = {b.n1, L(b.n1, {bi, si, ek})};
            q.B = {dqkv[cq], L(dqkv[cq], {bi, si, hj, 0})};
            q.C = {gwqkv, L(gwqkv, {ek, cq, hj, 0})};
            q.beta = (ti > 0 || later_mb) ? 1.f : 0.f;
            qs.push_back(q);
          }
      TRY(submit_gemm_batch(ctx, "qkv_dw", qs, true));
      for (int64_t ek = 0; ek < NE; ++ek) {
        std::vector<TileRef> As, Bs;
        for (int cq = 0; cq < 3; ++cq)
          for (int64_t hj = 0; hj < NH; ++hj) {
            As.push_back({dqkv[cq], L(dqkv[cq], {bi, si, hj, 0})});
            Bs.push_back({wqkv, L(wqkv, {ek, cq, hj, 0})});
          }
        TRY(submit_ksum_tb(ctx, "qkv_dx", {g->dn, L(g->dn, {bi, si, ek})}, As, Bs));
      }
      TRY(rms_backward(g, g->dn, b.h_in, an, b.ln1, g->dh, 1, g->G[g->lidx(l, ANORM)], bi, si));
    }
  return TT_OK;
}

// One minibatch: forward, loss, backward and (if do_update) AdamW. Minibatch
// `micro` of `n_micro` accumulates into the gradients and the loss of the
// earlier ones (micro > 0); the loss is scaled for the mean over all of them.
static int submit_step(tt_gpt2* g, const int32_t* tokens, const tt_adamw_hparams* hp, int do_update, int micro,
                       int n_micro) {
  tt_ctx* ctx = g->ctx;
  const int64_t t0 = ctx->next_id;
  const tt_gpt2_config& c = g->c;
  const int64_t B = c.batch, T = c.seq, hd = g->hd, V = c.vocab;
  const int64_t bt = g->t.batch, sq = g->t.seq, ht = g->t.head, rows = g->rows;
  const int64_t NE = g->NE, NI = g->NI, NH = g->NH, NV = g->NV;
  const float scale = 1.f / std::sqrt((float)hd);
  const float inv_n = 1.f / (float)(B * T * n_micro);
  const bool later_mb = micro > 0;  // gradients and loss already hold earlier minibatches

  // ---- inputs: copy the token windows, split into ids/labels, index for the embedding backward
  {
    const TileArg T[1] = {{g->tokens, 0}};
    const tt_op_copy sc{tokens};
    TRY(submit_op(ctx, TT_OP_COPY_IN, T, 1, &sc, sizeof(sc), "tokens", false));
  }
  for (int64_t bi = 0; bi < g->nb; ++bi)
    for (int64_t si = 0; si < g->ns; ++si) {
      const int64_t li = L(g->ids, {bi, si});
      const TileArg sp[3] = {{g->tokens, 0}, {g->ids, li}, {g->labels, li}};
      TRY(submit_op(ctx, TT_OP_SPLIT_TOKENS, sp, 3, nullptr, 0, "split", false));
      const TileArg ix[3] = {{g->ids, li}, {g->sorted, li}, {g->perm, li}};
      TRY(submit_op(ctx, TT_OP_EMBEDDING_INDEX, ix, 3, nullptr, 0, "emb_index", false));
    }

  // The inputs' tasks go to the GPU now, so it starts on this step while the
  // host infers the dependencies of the rest (with a large window it would
  // otherwise wait for the whole step's submission), and the copy of the
  // caller's token buffer is queued before this call returns. The inputs
  // touch no pinned-host tile, so the residency plan of the rest still
  // covers the whole step.
  TRY(ctx->flush());

  // ---- embedding forward
  tt_tensor* h0 = c.n_layer ? g->blk[0].h_in : g->h_last;
  for (int64_t bi = 0; bi < g->nb; ++bi)
    for (int64_t si = 0; si < g->ns; ++si)
      for (int64_t e = 0; e < NE; ++e) {
        tt_tensor* wte = g->P[0];
        std::vector<TileArg> T = {{g->ids, L(g->ids, {bi, si})}};
        if (!g->llama) T.push_back({g->P[1], L(g->P[1], {si, e})});  // positions (GPT2)
        T.push_back({h0, L(h0, {bi, si, e})});
        for (int64_t v = 0; v < NV; ++v) T.push_back({wte, L(wte, {v, e})});
        const tt_op_embedding sc{sq};
        TRY(submit_op(ctx, g->llama ? TT_OP_EMBEDDING_TOKEN_FWD : TT_OP_EMBEDDING_FWD, T.data(), (int)T.size(), &sc,
                      sizeof(sc), "emb_fwd", false));
      }

  // ---- blocks forward
  for (int l = 0; l < c.n_layer; ++l) {
    if (g->llama) {
      TRY(llama_block_forward(g, l));
      continue;
    }
    BlockT& b = g->blk[l];
    tt_tensor* hout = (l + 1 < c.n_layer) ? g->blk[l + 1].h_in : g->h_last;
    tt_tensor *ln1g = g->P[g->pidx(l, LN1G)], *ln1b = g->P[g->pidx(l, LN1B)];
    tt_tensor *wqkv = g->P[g->pidx(l, WQKV)], *bqkv = g->P[g->pidx(l, BQKV)];
    tt_tensor *wo = g->P[g->pidx(l, WO)], *bo = g->P[g->pidx(l, BO)];
    tt_tensor *ln2g = g->P[g->pidx(l, LN2G)], *ln2b = g->P[g->pidx(l, LN2B)];
    tt_tensor *wfc = g->P[g->pidx(l, WFC)], *bfc = g->P[g->pidx(l, BFC)];
    tt_tensor *wp = g->P[g->pidx(l, WP)], *bp = g->P[g->pidx(l, BP)];
    tt_tensor* qkv[3] = {b.q, b.k, b.v};
    for (int64_t bi = 0; bi < g->nb; ++bi)
      for (int64_t si = 0; si < g->ns; ++si) {
        const int64_t ti = bi + g->nb * si;
        TRY(ln_forward(g, b.h_in, ln1g, ln1b, b.ln1, b.n1, bi, si));
        for (int cq = 0; cq < 3; ++cq)
          for (int64_t hj = 0; hj < NH; ++hj) {
            const TileRef C = {qkv[cq], L(qkv[cq], {bi, si, hj, 0})}, bias = {bqkv, L(bqkv, {cq, hj, 0})};
            if (use_ksum("qkv", C, 0, {b.n1, L(b.n1, {bi, si, 0})})) {
              std::vector<TileRef> As, Bs;
              for (int64_t ek = 0; ek < NE; ++ek) {
                As.push_back({b.n1, L(b.n1, {bi, si, ek})});
                Bs.push_back({wqkv, L(wqkv, {ek, cq, hj, 0})});
              }
              TRY(submit_ksum(ctx, "qkv", 0, C, As, Bs, TT_EPI_BIAS, bias));
              continue;
            }
            for (int64_t ek = 0; ek < NE; ++ek) {
              Gemm q;
              q.A = {b.n1, L(b.n1, {bi, si, ek})};
              q.B = {wqkv, L(wqkv, {ek, cq, hj, 0})};
              q.C = C;
              q.beta = ek > 0 ? 1.f : 0.f;
              if (ek == NE - 1) {
                q.epi = TT_EPI_BIAS;
                q.bias = bias;
              }
              TRY(submit_gemm(ctx, "qkv", q));
            }
          }
      }
    TRY(attention_forward(g, b));
    for (int64_t bi = 0; bi < g->nb; ++bi)
      for (int64_t si = 0; si < g->ns; ++si) {
        const int64_t ti = bi + g->nb * si;
        // h_mid = h_in + O W_o + b_o
        for (int64_t ej = 0; ej < NE; ++ej) {
          if (use_ksum("attn_proj", {b.h_mid, L(b.h_mid, {bi, si, ej})}, 0, {b.o, L(b.o, {bi, si, 0, 0})})) {
            std::vector<TileRef> As, Bs;
            for (int64_t hk = 0; hk < NH; ++hk) {
              As.push_back({b.o, L(b.o, {bi, si, hk, 0})});
              Bs.push_back({wo, L(wo, {hk, 0, ej})});
            }
            TRY(submit_ksum(ctx, "attn_proj", 0, {b.h_mid, L(b.h_mid, {bi, si, ej})}, As, Bs,
                            TT_EPI_RES | TT_EPI_BIAS, {bo, ej}, {b.h_in, L(b.h_in, {bi, si, ej})}));
            continue;
          }
          for (int64_t hk = 0; hk < NH; ++hk) {
            Gemm q;
            q.A = {b.o, L(b.o, {bi, si, hk, 0})};
            q.B = {wo, L(wo, {hk, 0, ej})};
            q.C = {b.h_mid, L(b.h_mid, {bi, si, ej})};
            q.beta = hk > 0 ? 1.f : 0.f;
            if (hk == 0) {
              q.epi |= TT_EPI_RES;
              q.res = {b.h_in, L(b.h_in, {bi, si, ej})};
            }
            if (hk == NH - 1) {
              q.epi |= TT_EPI_BIAS;
              q.bias = {bo, ej};
            }
            TRY(submit_gemm(ctx, "attn_proj", q));
          }
        }
        TRY(ln_forward(g, b.h_mid, ln2g, ln2b, b.ln2, b.n2, bi, si));
        // g = gelu(n2 W_fc + b_fc), pre-activation kept in u
        for (int64_t ij = 0; ij < NI; ++ij) {
          if (use_ksum("fc", {b.g, L(b.g, {bi, si, ij})}, 0, {b.n2, L(b.n2, {bi, si, 0})})) {
            std::vector<TileRef> As, Bs;
            for (int64_t ek = 0; ek < NE; ++ek) {
              As.push_back({b.n2, L(b.n2, {bi, si, ek})});
              Bs.push_back({wfc, L(wfc, {ek, ij})});
            }
            TRY(submit_ksum(ctx, "fc", 0, {b.g, L(b.g, {bi, si, ij})}, As, Bs, TT_EPI_GELU | TT_EPI_BIAS, {bfc, ij},
                            {}, {b.u, L(b.u, {bi, si, ij})}));
            continue;
          }
          for (int64_t ek = 0; ek < NE; ++ek) {
            Gemm q;
            q.A = {b.n2, L(b.n2, {bi, si, ek})};
            q.B = {wfc, L(wfc, {ek, ij})};
            q.beta = ek > 0 ? 1.f : 0.f;
            if (ek == NE - 1) {
              q.C = {b.g, L(b.g, {bi, si, ij})};
              q.epi = TT_EPI_GELU | TT_EPI_BIAS;
              q.bias = {bfc, ij};
              q.aux = {b.u, L(b.u, {bi, si, ij})};
            } else {
              q.C = {b.u, L(b.u, {bi, si, ij})};
            }
            TRY(submit_gemm(ctx, "fc", q));
          }
        }
        // h_out = h_mid + g W_p + b_p
        for (int64_t ej = 0; ej < NE; ++ej) {
          if (use_ksum("mlp_proj", {hout, L(hout, {bi, si, ej})}, 0, {b.g, L(b.g, {bi, si, 0})})) {
            std::vector<TileRef> As, Bs;
            for (int64_t ik = 0; ik < NI; ++ik) {
              As.push_back({b.g, L(b.g, {bi, si, ik})});
              Bs.push_back({wp, L(wp, {ik, ej})});
            }
            TRY(submit_ksum(ctx, "mlp_proj", 0, {hout, L(hout, {bi, si, ej})}, As, Bs, TT_EPI_RES | TT_EPI_BIAS,
                            {bp, ej}, {b.h_mid, L(b.h_mid, {bi, si, ej})}));
            continue;
          }
          for (int64_t ik = 0; ik < NI; ++ik) {
            Gemm q;
            q.A = {b.g, L(b.g, {bi, si, ik})};
            q.B = {wp, L(wp, {ik, ej})};
            q.C = {hout, L(hout, {bi, si, ej})};
            q.beta = ik > 0 ? 1.f : 0.f;
            if (ik == 0) {
              q.epi |= TT_EPI_RES;
              q.res = {b.h_mid, L(b.h_mid, {bi, si, ej})};
            }
            if (ik == NI - 1) {
              q.epi |= TT_EPI_BIAS;
              q.bias = {bp, ej};
            }
            TRY(submit_gemm(ctx, "mlp_proj", q));
          }
        }
      }
  }

  // ---- final LayerNorm (RMSNorm), head (tied to wte for GPT2), cross-entropy
  tt_tensor* lnfg = g->P[g->llama ? g->norm_f() : g->lnf_g()];
  tt_tensor* lnfb = g->llama ? nullptr : g->P[g->lnf_g() + 1];
  tt_tensor* wte = g->P[g->head_w()];  // the head's weight
  for (int64_t bi = 0; bi < g->nb; ++bi)
    for (int64_t si = 0; si < g->ns; ++si) {
      const int64_t ti = bi + g->nb * si;
      if (g->llama) TRY(rms_forward(g, g->h_last, lnfg, g->lnf, g->nf, bi, si));
      else TRY(ln_forward(g, g->h_last, lnfg, lnfb, g->lnf, g->nf, bi, si));
      // z_v = nf wte_v^T for every vocab tile v: per embd tile, one batch
      // of equal-shape products (tile_gemm_batch), accumulating over embd
      // tiles; the last embd tile's batch also takes the cross-entropy
      // statistics of the finished logits in its epilogue (per row and
      // 64-column group: max, sum exp, target logit), so the logits are not
      // read again for them
      tt_tensor *z = g->z, *parts = g->ce_parts;
      const int64_t ll = L(g->labels, {bi, si});
      const bool ksum = head_ksum(NE);
      const bool fused = head_xstats() && !ksum;
      if (ksum) {
        // z_v = sum over the embd tiles of nf_e wte_v,e^T: one long-K task
        // per vocab tile
        for (int64_t vj = 0; vj < NV; ++vj) {
          std::vector<TileRef> As, Bs;
          for (int64_t ek = 0; ek < NE; ++ek) {
            As.push_back({g->nf, L(g->nf, {bi, si, ek})});
            Bs.push_back({wte, L(wte, {vj, ek})});
          }
          TRY(submit_ksum(ctx, "head", 1, {g->z, L(g->z, {bi, si, vj})}, As, Bs));
        }
      }
      for (int64_t ek = 0; ek < (ksum ? 0 : NE); ++ek) {
        std::vector<Gemm> qs;
        for (int64_t vj = 0; vj < NV; ++vj) {
          Gemm q;
          q.tb = 1;
          q.A = {g->nf, L(g->nf, {bi, si, ek})};
          q.B = {wte, L(wte, {vj, ek})};
          q.C = {g->z, L(g->z, {bi, si, vj})};
          q.beta = ek > 0 ? 1.f : 0.f;
          qs.push_back(q);
        }
        if (fused && ek == NE - 1) {
          // tasks of up to 96 consecutive vocab tiles and 1 GiB of logits
          const int64_t tile_bytes = g->rows * std::min<int64_t>(g->t.vocab, c.vocab) * (int64_t)sizeof(float);
          const int64_t per = std::max<int64_t>(1, std::min<int64_t>(96, (int64_t(1) << 30) / tile_bytes));
          for (int64_t v0 = 0; v0 < NV; v0 += per) {
            const int64_t v1 = std::min(NV, v0 + per);
            std::vector<TileArg> T;
            for (int64_t vj = v0; vj < v1; ++vj) {
              T.push_back(ta(qs[vj].A));
              T.push_back(ta(qs[vj].B));
              T.push_back(ta(qs[vj].C));
            }
            T.push_back({g->labels, ll});
            for (int64_t vj = v0; vj < v1; ++vj) T.push_back({parts, L(parts, {vj, ti, 0})});
            const tt_op_gemm sc{0, 1, TT_EPI_XSTATS, 1.f, qs[0].beta, 0};
            TRY(submit_op(ctx, TT_OP_GEMM_BATCH, T.data(), (int)T.size(), &sc, sizeof(sc), "head", false));
          }
        } else {
          TRY(submit_gemm_batch(ctx, "head", qs));
        }
      }
      if (!fused) {
        // per-vocab-tile (max, sum exp, target logit) partials: one task and
        // launch over all vocab tiles of the token tile (tile_xentropy_multi)
        std::vector<TileArg> T = {{g->labels, ll}};
        for (int64_t vj = 0; vj < NV; ++vj) T.push_back({z, L(z, {bi, si, vj})});
        for (int64_t vj = 0; vj < NV; ++vj) T.push_back({parts, L(parts, {vj, ti, 0})});
        TRY(submit_op(ctx, TT_OP_XENTROPY_STATS, T.data(), (int)T.size(), nullptr, 0, "ce_stats", false));
      }
      {
        std::vector<TileArg> T = {{g->ce_lse, ti}, {g->row_loss, ti}};
        for (int64_t vj = 0; vj < NV; ++vj) T.push_back({parts, L(parts, {vj, ti, 0})});
        const tt_op_xe_groups gs{c.vocab, std::min<int64_t>(g->t.vocab, c.vocab), 64};
        TRY(submit_op(ctx, TT_OP_XENTROPY_MERGE, T.data(), (int)T.size(), fused ? &gs : nullptr,
                      fused ? sizeof(gs) : 0, "ce_merge", false));
      }
      {
        const TileArg T[2] = {{g->row_loss, ti}, {g->loss, 0}};
        const tt_op_xentropy sc{ti > 0 || later_mb, inv_n};
        TRY(submit_op(ctx, TT_OP_XENTROPY_LOSS, T, 2, &sc, sizeof(sc), "ce_loss", false));
      }
      {
        // dz in place of the logits, all vocab tiles of the token tile in one
        // task and launch
        std::vector<TileArg> T = {{g->labels, ll}, {g->ce_lse, ti}};
        for (int64_t vj = 0; vj < NV; ++vj) T.push_back({z, L(z, {bi, si, vj})});
        const tt_op_xentropy sc{0, inv_n};
        TRY(submit_op(ctx, TT_OP_XENTROPY_GRAD, T.data(), (int)T.size(), &sc, sizeof(sc), "ce_grad", false));
      }
    }

  // ---- AdamW, one task per parameter tile, submitted as soon as the
  // tile's gradient is final (after the backward of the parameter's own
  // layer): the update overlaps the rest of the backward and finds p and g
  // still resident; the result is the same as updating at the end, since no
  // later task of the step reads these parameters
  // Small tiles (LayerNorm gains, biases) would each be a launch of a few
  // microseconds: tiles of the given parameters are packed into tasks of up
  // to TT_ADAMW_MAX_TILES tiles and 16 Mi elements, one launch each (a
  // GPT2-small layer's 7.1 M parameters are one launch: 0.75 -> 0.69 ms per
  // step against 4 Mi).
  tt_tensor *stp = g->step, *bc = g->bc;
  const tt_adamw_hparams h = *hp;
  auto adamw_of = [&](std::initializer_list<size_t> params) -> int {
    if (!do_update) return TT_OK;
    struct Item {
      size_t i;
      int64_t lt, n;
    };
    std::vector<Item> items;
    for (size_t i : params)
      for (int64_t lt = 0; lt < g->P[i]->ntiles; ++lt) items.push_back({i, lt, g->P[i]->tile_elems(lt)});
    // with pinned-host homes a task's tiles must fit the device arena (p, g,
    // m and v of every tile): a group then takes at most an eighth of it
    int64_t max_elems = int64_t(16) << 20;
    if (g->param_home != TT_HOME_DEVICE && ctx->budget > 0)
      max_elems = std::min<int64_t>(max_elems, (int64_t)(ctx->budget / (8 * 4 * sizeof(float))));
    size_t k = 0;
    while (k < items.size()) {
      std::vector<Item> grp;
      int64_t elems = 0;
      while (k < items.size() && (int)grp.size() < TT_ADAMW_MAX_TILES &&
             (grp.empty() || elems + items[k].n <= max_elems)) {
        elems += items[k].n;
        grp.push_back(items[k++]);
      }
      std::vector<TileArg> T;
      const tt_op_optim sc{h.lr, h.beta1, h.beta2, h.eps, h.weight_decay};
      if (h.optimizer == TT_OPT_SGD) {  // p -= lr g: the moments are not touched
        for (const Item& it : grp) {
          T.push_back({g->P[it.i], it.lt});
          T.push_back({g->G[it.i], it.lt});
        }
        TRY(submit_op(ctx, TT_OP_SGD, T.data(), (int)T.size(), &sc, sizeof(sc), "sgd", false));
        continue;
      }
      T.push_back({bc, 0});
      for (const Item& it : grp) {
        T.push_back({g->P[it.i], it.lt});
        T.push_back({g->G[it.i], it.lt});
        T.push_back({g->M[it.i], it.lt});
        T.push_back({g->Vv[it.i], it.lt});
      }
      TRY(submit_op(ctx, TT_OP_ADAMW, T.data(), (int)T.size(), &sc, sizeof(sc), "adamw", false));
    }
    return TT_OK;
  };
  if (do_update && h.optimizer == TT_OPT_ADAMW) {
    const TileArg T[2] = {{stp, 0}, {bc, 0}};
    const tt_op_optim sc{h.lr, hp->beta1, hp->beta2, h.eps, h.weight_decay};
    TRY(submit_op(ctx, TT_OP_ADAMW_ADVANCE, T, 2, &sc, sizeof(sc), "adam_step", false));
  }

  // ---- backward: head (dz is in place of the logits)
  // dwte (head part; dw_head when untied) = sum over token tiles of dz^T nf:
  // per (embd tile, token tile), one batch of equal-shape products over the
  // vocab tiles
  tt_tensor* gwte = g->G[g->head_w()];
  for (int64_t ek = 0; ek < NE; ++ek)
    for (int64_t si = 0; si < g->ns; ++si)
      for (int64_t bi = 0; bi < g->nb; ++bi) {
        const int64_t ti = bi + g->nb * si;
        std::vector<Gemm> qs;
        for (int64_t vj = 0; vj < NV; ++vj) {
          Gemm q;
          q.ta = 1;
          q.A = {g->z, L(g->z, {bi, si, vj})};
          q.B = {g->nf, L(g->nf, {bi, si, ek})};
          q.C = {gwte, L(gwte, {vj, ek})};
          q.beta = (ti > 0 || later_mb) ? 1.f : 0.f;
          qs.push_back(q);
        }
        TRY(submit_gemm_batch(ctx, "head_dw", qs));
      }
  // dnf = sum over vocab tiles of dz wte: one task per (token tile, embd
  // tile), one long-K product over every vocab tile (tile_gemm_ksum), instead
  // of a chain of accumulating GEMMs that each read and write dnf
  for (int64_t si = 0; si < g->ns; ++si)
    for (int64_t bi = 0; bi < g->nb; ++bi)
      for (int64_t ek = 0; ek < NE; ++ek) {
        std::vector<TileArg> T = {{g->dnf, L(g->dnf, {bi, si, ek})}};
        for (int64_t vj = 0; vj < NV; ++vj) {
          T.push_back({g->z, L(g->z, {bi, si, vj})});
          T.push_back({wte, L(wte, {vj, ek})});
        }
        const tt_op_gemm sc{0, 0, TT_EPI_NONE, 1.f, 0.f, 1};
        TRY(submit_op(ctx, TT_OP_GEMM_KSUM, T.data(), (int)T.size(), &sc, sizeof(sc), "head_dx", false));
      }
  if (g->llama) TRY(adamw_of({(size_t)g->head_w()}));  // the untied head's gradient is final
  // zero the LayerNorm and position gradients, which accumulate (over
  // token tiles, and over minibatches after the first); LLaMA: the RMSNorm
  // gains' and the token table's (no head part writes it first)
  if (!later_mb && g->llama) {
    std::vector<TileRef> zero;
    for (int l = 0; l < c.n_layer; ++l)
      for (int w : {ANORM, MNORM})
        for (int64_t e = 0; e < NE; ++e) zero.push_back({g->G[g->lidx(l, w)], e});
    for (int64_t e = 0; e < NE; ++e) zero.push_back({g->G[g->norm_f()], e});
    for (int64_t lt = 0; lt < g->G[0]->ntiles; ++lt) zero.push_back({g->G[0], lt});
    TRY(fill_tasks(g, zero, 0.f));
  } else if (!later_mb) {
    std::vector<TileRef> zero;
    for (int l = 0; l < c.n_layer; ++l)
      for (int w : {LN1G, LN1B, LN2G, LN2B})
        for (int64_t e = 0; e < NE; ++e) zero.push_back({g->G[g->pidx(l, w)], e});
    for (int64_t e = 0; e < NE; ++e) {
      zero.push_back({g->G[g->lnf_g()], e});
      zero.push_back({g->G[g->lnf_g() + 1], e});
    }
    for (int64_t lt = 0; lt < g->G[1]->ntiles; ++lt) zero.push_back({g->G[1], lt});
    TRY(fill_tasks(g, zero, 0.f));
  }
  for (int64_t bi = 0; bi < g->nb; ++bi)
    for (int64_t si = 0; si < g->ns; ++si) {
      if (g->llama) TRY(rms_backward(g, g->dnf, g->h_last, lnfg, g->lnf, g->dh, 0, g->G[g->norm_f()], bi, si));
      else
        TRY(ln_backward(g, g->dnf, g->h_last, lnfg, g->lnf, g->dh, 0, g->G[g->lnf_g()], g->G[g->lnf_g() + 1], bi,
                        si));
    }
  if (g->llama) TRY(adamw_of({(size_t)g->norm_f()}));
  else TRY(adamw_of({(size_t)g->lnf_g(), (size_t)g->lnf_g() + 1}));

  // bias gradients of a row of tiles (token tile (bi, si), n feature
  // tiles): up to 16 tiles per task, one pair of launches each
  auto colsum_row = [&](tt_tensor* x, tt_tensor* out, int64_t n, int64_t bi, int64_t si, int beta) -> int {
    for (int64_t f0 = 0; f0 < n; f0 += 16) {
      std::vector<TileRef> xs, os;
      for (int64_t f = f0; f < std::min(n, f0 + 16); ++f) {
        xs.push_back({x, L(x, {bi, si, f})});
        os.push_back({out, f});
      }
      TRY(colsum_task(ctx, xs, os, beta));
    }
    return TT_OK;
  };

  // ---- blocks backward
  for (int l = c.n_layer - 1; l >= 0; --l) {
    if (g->llama) {
      TRY(llama_block_backward(g, l, later_mb));
      const size_t p0 = g->lidx(l, 0);
      TRY(adamw_of({p0 + ANORM, p0 + MNORM, p0 + LQKV, p0 + LWO, p0 + LGATE, p0 + LUP, p0 + LDOWN}));
      continue;
    }
    BlockT& b = g->blk[l];
    tt_tensor *ln1g = g->P[g->pidx(l, LN1G)], *wqkv = g->P[g->pidx(l, WQKV)], *wo = g->P[g->pidx(l, WO)];
    tt_tensor *ln2g = g->P[g->pidx(l, LN2G)], *wfc = g->P[g->pidx(l, WFC)], *wp = g->P[g->pidx(l, WP)];
    tt_tensor *gwqkv = g->G[g->pidx(l, WQKV)], *gbqkv = g->G[g->pidx(l, BQKV)];
    tt_tensor *gwo = g->G[g->pidx(l, WO)], *gbo = g->G[g->pidx(l, BO)];
    tt_tensor *gwfc = g->G[g->pidx(l, WFC)], *gbfc = g->G[g->pidx(l, BFC)];
    tt_tensor *gwp = g->G[g->pidx(l, WP)], *gbp = g->G[g->pidx(l, BP)];
    tt_tensor* dqkv[3] = {g->dq, g->dk, g->dv};
    tt_tensor* qkv[3] = {b.q, b.k, b.v};
    // MLP: h_out = h_mid + gelu(u) W_p + b_p
    for (int64_t si = 0; si < g->ns; ++si)
      for (int64_t bi = 0; bi < g->nb; ++bi) {
        const int64_t ti = bi + g->nb * si;
        // weight gradients of every (inner, embd) tile pair: one batched task
        // (split-K over the stream's workspace when the products are few)
        {
          std::vector<Gemm> qs;
          for (int64_t ej = 0; ej < NE; ++ej)
            for (int64_t ik = 0; ik < NI; ++ik) {
              Gemm q;
              q.ta = 1;
              q.A = {b.g, L(b.g, {bi, si, ik})};
              q.B = {g->dh, L(g->dh, {bi, si, ej})};
              q.C = {gwp, L(gwp, {ik, ej})};
              q.beta = (ti > 0 || later_mb) ? 1.f : 0.f;
              qs.push_back(q);
            }
          TRY(submit_gemm_batch(ctx, "mlp_proj_dw", qs, true));
        }
        TRY(colsum_row(g->dh, gbp, NE, bi, si, ti > 0 || later_mb));
        for (int64_t ik = 0; ik < NI; ++ik) {
          if (use_ksum("mlp_proj_dx", {g->dgu, L(g->dgu, {bi, si, ik})}, 1, {g->dh, L(g->dh, {bi, si, 0})})) {
            std::vector<TileRef> As, Bs;
            for (int64_t ej = 0; ej < NE; ++ej) {
              As.push_back({g->dh, L(g->dh, {bi, si, ej})});
              Bs.push_back({wp, L(wp, {ik, ej})});
            }
            TRY(submit_ksum(ctx, "mlp_proj_dx", 1, {g->dgu, L(g->dgu, {bi, si, ik})}, As, Bs, TT_EPI_GELU_BWD, {}, {},
                            {b.u, L(b.u, {bi, si, ik})}));
            continue;
          }
          for (int64_t ej = 0; ej < NE; ++ej) {
            Gemm q;
            q.tb = 1;
            q.A = {g->dh, L(g->dh, {bi, si, ej})};
            q.B = {wp, L(wp, {ik, ej})};
            q.C = {g->dgu, L(g->dgu, {bi, si, ik})};
            q.beta = ej > 0 ? 1.f : 0.f;
            if (ej == NE - 1) {
              q.epi = TT_EPI_GELU_BWD;
              q.aux = {b.u, L(b.u, {bi, si, ik})};
            }
            TRY(submit_gemm(ctx, "mlp_proj_dx", q));
          }
        }
        {
          std::vector<Gemm> qs;
          for (int64_t ik = 0; ik < NI; ++ik)
            for (int64_t ek = 0; ek < NE; ++ek) {
              Gemm q;
              q.ta = 1;
              q.A = {b.n2, L(b.n2, {bi, si, ek})};
              q.B = {g->dgu, L(g->dgu, {bi, si, ik})};
              q.C = {gwfc, L(gwfc, {ek, ik})};
              q.beta = (ti > 0 || later_mb) ? 1.f : 0.f;
              qs.push_back(q);
            }
          TRY(submit_gemm_batch(ctx, "fc_dw", qs, true));
        }
        TRY(colsum_row(g->dgu, gbfc, NI, bi, si, ti > 0 || later_mb));
        // (a chain of accumulating GEMMs: as one long-K task per embd tile it
        // measured slower on the wide model, 65 -> 71 ms per step)
        for (int64_t ek = 0; ek < NE; ++ek) {
          if (use_ksum("fc_dx", {g->dn, L(g->dn, {bi, si, ek})}, 1, {g->dgu, L(g->dgu, {bi, si, 0})})) {
            std::vector<TileRef> As, Bs;
            for (int64_t ik = 0; ik < NI; ++ik) {
              As.push_back({g->dgu, L(g->dgu, {bi, si, ik})});
              Bs.push_back({wfc, L(wfc, {ek, ik})});
            }
            TRY(submit_ksum(ctx, "fc_dx", 1, {g->dn, L(g->dn, {bi, si, ek})}, As, Bs));
            continue;
          }
          for (int64_t ik = 0; ik < NI; ++ik) {
            Gemm q;
            q.tb = 1;
            q.A = {g->dgu, L(g->dgu, {bi, si, ik})};
            q.B = {wfc, L(wfc, {ek, ik})};
            q.C = {g->dn, L(g->dn, {bi, si, ek})};
            q.beta = ik > 0 ? 1.f : 0.f;
            TRY(submit_gemm(ctx, "fc_dx", q));
          }
        }
        TRY(ln_backward(g, g->dn, b.h_mid, ln2g, b.ln2, g->dh, 1, g->G[g->pidx(l, LN2G)], g->G[g->pidx(l, LN2B)], bi,
                        si));
        // attention projection: h_mid = h_in + O W_o + b_o
        {
          std::vector<Gemm> qs;
          for (int64_t ej = 0; ej < NE; ++ej)
            for (int64_t hk = 0; hk < NH; ++hk) {
              Gemm q;
              q.ta = 1;
              q.A = {b.o, L(b.o, {bi, si, hk, 0})};
              q.B = {g->dh, L(g->dh, {bi, si, ej})};
              q.C = {gwo, L(gwo, {hk, 0, ej})};
              q.beta = (ti > 0 || later_mb) ? 1.f : 0.f;
              qs.push_back(q);
            }
          TRY(submit_gemm_batch(ctx, "attn_proj_dw", qs, true));
        }
        TRY(colsum_row(g->dh, gbo, NE, bi, si, ti > 0 || later_mb));
        for (int64_t hk = 0; hk < NH; ++hk) {
          if (use_ksum("attn_proj_dx", {g->dO, L(g->dO, {bi, si, hk, 0})}, 1, {g->dh, L(g->dh, {bi, si, 0})})) {
            std::vector<TileRef> As, Bs;
            for (int64_t ej = 0; ej < NE; ++ej) {
              As.push_back({g->dh, L(g->dh, {bi, si, ej})});
              Bs.push_back({wo, L(wo, {hk, 0, ej})});
            }
            TRY(submit_ksum(ctx, "attn_proj_dx", 1, {g->dO, L(g->dO, {bi, si, hk, 0})}, As, Bs));
            continue;
          }
          for (int64_t ej = 0; ej < NE; ++ej) {
            Gemm q;
            q.tb = 1;
            q.A = {g->dh, L(g->dh, {bi, si, ej})};
            q.B = {wo, L(wo, {hk, 0, ej})};
            q.C = {g->dO, L(g->dO, {bi, si, hk, 0})};
            q.beta = ej > 0 ? 1.f : 0.f;
            TRY(submit_gemm(ctx, "attn_proj_dx", q));
          }
        }
      }
    TRY(attention_backward(g, b));
    // QKV projection backward
    for (int64_t si = 0; si < g->ns; ++si)
      for (int64_t bi = 0; bi < g->nb; ++bi) {
        const int64_t ti = bi + g->nb * si;
        // the q, k and v weight gradients of every (head, embd) tile pair:
        // independent products of one K (the token tile), one batched task
        // (split-K over the stream's workspace when they are few)
        std::vector<Gemm> qs;
        for (int cq = 0; cq < 3; ++cq)
          for (int64_t hj = 0; hj < NH; ++hj)
            for (int64_t ek = 0; ek < NE; ++ek) {
              Gemm q;
              q.ta = 1;
              q.A = {b.n1, L(b.n1, {bi, si, ek})};
              q.B = {dqkv[cq], L(dqkv[cq], {bi, si, hj, 0})};
              q.C = {gwqkv, L(gwqkv, {ek, cq, hj, 0})};
              q.beta = (ti > 0 || later_mb) ? 1.f : 0.f;
              qs.push_back(q);
            }
        TRY(submit_gemm_batch(ctx, "qkv_dw", qs, true));
        // the q, k and v bias gradients of every head tile: one task, one
        // pair of launches (tile_reduce_rows_multi), up to 15 tiles each
        {
          std::vector<TileRef> xs, os;
          for (int cq = 0; cq < 3; ++cq)
            for (int64_t hj = 0; hj < NH; ++hj) {
              xs.push_back({dqkv[cq], L(dqkv[cq], {bi, si, hj, 0})});
              os.push_back({gbqkv, L(gbqkv, {cq, hj, 0})});
            }
          for (size_t u0 = 0; u0 < xs.size(); u0 += 15) {
            const size_t u1 = std::min(xs.size(), u0 + 15);
            TRY(colsum_task(ctx, {xs.begin() + u0, xs.begin() + u1}, {os.begin() + u0, os.begin() + u1},
                            ti > 0 || later_mb));
          }
        }
        // dn = sum over (q|k|v, head tile) of dqkv W_qkv^T: one task per embd
        // tile, one long-K product over the 3 * NH pairs (tile_gemm_ksum)
        for (int64_t ek = 0; ek < NE; ++ek) {
          std::vector<TileRef> As, Bs;
          for (int cq = 0; cq < 3; ++cq)
            for (int64_t hj = 0; hj < NH; ++hj) {
              As.push_back({dqkv[cq], L(dqkv[cq], {bi, si, hj, 0})});
              Bs.push_back({wqkv, L(wqkv, {ek, cq, hj, 0})});
            }
          TRY(submit_ksum_tb(ctx, "qkv_dx", {g->dn, L(g->dn, {bi, si, ek})}, As, Bs));
        }
        TRY(ln_backward(g, g->dn, b.h_in, ln1g, b.ln1, g->dh, 1, g->G[g->pidx(l, LN1G)], g->G[g->pidx(l, LN1B)], bi,
                        si));
      }
    (void)qkv;
    {
      const size_t p0 = g->pidx(l, 0);
      TRY(adamw_of({p0 + LN1G, p0 + LN1B, p0 + BQKV, p0 + BO, p0 + LN2G, p0 + LN2B, p0 + BFC, p0 + BP, p0 + WQKV,
                    p0 + WO, p0 + WFC, p0 + WP}));
    }
  }

  // ---- embedding backward: token rows into dwte (after its head part), positions into dwpe.
  // In HBM the dwte tiles of one embd column are one contiguous [V, et] slab
  // (first grid axis fastest), so one launch per (embd tile, token tile)
  // covers every vocab tile; staged pinned tiles are separate, one launch each.
  for (int64_t ek = 0; ek < NE; ++ek)
    for (int64_t si = 0; si < g->ns; ++si)
      for (int64_t bi = 0; bi < g->nb; ++bi) {
        const int64_t li = L(g->sorted, {bi, si});
        const TileArg head[3] = {{g->dh, L(g->dh, {bi, si, ek})}, {g->sorted, li}, {g->perm, li}};
        const tt_op_embedding sc{sq};
        // in HBM the dwte tiles of one embd column are one contiguous slab:
        // one task and launch over every vocab tile; staged pinned tiles are
        // separate, one task per vocab tile
        tt_tensor* gtok = g->G[0];
        const int64_t per = gtok->home == TT_HOME_DEVICE ? NV : 1;
        for (int64_t v0 = 0; v0 < NV; v0 += per) {
          std::vector<TileArg> T(head, head + 3);
          for (int64_t vj = v0; vj < v0 + per; ++vj) T.push_back({gtok, L(gtok, {vj, ek})});
          TRY(submit_op(ctx, TT_OP_EMBEDDING_BWD, T.data(), (int)T.size(), &sc, sizeof(sc), "emb_dw", false));
        }
      }
  for (int64_t si = 0; si < g->ns && !g->llama; ++si)
    for (int64_t ek = 0; ek < NE; ++ek)
      for (int64_t bi = 0; bi < g->nb; ++bi) {
        const TileArg T[2] = {{g->dh, L(g->dh, {bi, si, ek})}, {g->G[1], L(g->G[1], {si, ek})}};
        const tt_op_embedding sc{sq};
        TRY(submit_op(ctx, TT_OP_EMBEDDING_POS_BWD, T, 2, &sc, sizeof(sc), "emb_dpos", false));
      }

  // ---- AdamW of the embeddings (their gradients are final now)
  if (g->llama) TRY(adamw_of({0}));
  else TRY(adamw_of({1, 0}));
  g->last_tasks = ctx->next_id - t0;
  return ctx->flush();
}

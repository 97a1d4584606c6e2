// Host runtime of libcbd: slab arena, step planner and the C ABI (include/cbd.h).
//
// Page "Continuous Decode Batching - the transformer capture":
//  - section "1. Native station": one KV slab per live sequence in an arena
//    keyed by sequence id; admission = fresh slab at length 0; EOS = drop it;
//    the arena size caps concurrency and the caller queues the rest.
//  - section "decode_step_batch - paint-by-numbers": t_s is the sequence's
//    own length, captured once per step on the host and used for RoPE, the
//    append slot and the attention range; after the step t_s += 1.
// Page "Batching", section 6, item 3: a fork shares its parent's prefix blocks
// (kvslab_fork); the parent's memory stays allocated while forks read it.
// Failure containment (page "Batching", section 4.5): arguments are
// validated before anything is enqueued, so a rejected call changes no slab.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <string>
#include <vector>

#include "../../include/cbd.h"
#include "kernels.h"

using namespace cbd;

namespace {

constexpr int kGranuleTokens = 256;
constexpr int kStagingSlots = 4;
constexpr int kMaxParts = 4096;
constexpr int kExtraItems = kMaxParts + 64;

thread_local std::string g_err;

cbd_status fail(cbd_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

cbd_status hip_fail(hipError_t e, const char* what) {
  return fail(CBD_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define HIP_TRY(expr, what)                       \
  do {                                            \
    hipError_t e_ = (expr);                       \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)

struct Mat {
  const void* data;
  const void* aux;
};

struct LayerW {
  const uint16_t* attn_norm;
  Mat wq, wk, wv, wo;
  const uint16_t* ffn_norm;
  Mat wg, wu, wd;
};

struct Slab {
  int64_t off = 0;
  int32_t cap = 0;     // tokens the slab may hold (granule-rounded, clipped to the RoPE table)
  int32_t stride = 0;  // tokens per K or V region in the slab layout (granule-rounded)
  int32_t len = 0;
  int64_t gran_begin = 0, gran_count = 0;
  bool live = false;
  // shared prefix: keys [0, base) are read from slab `parent` (base a multiple of 32); a slab with
  // live forks that is freed stays allocated (zombie) until its last fork is freed
  int32_t base = 0;
  int32_t parent = -1;
  int32_t children = 0;
  bool zombie = false;
};

template <class T>
T* align_ptr(uint8_t*& p, size_t count) {
  p = reinterpret_cast<uint8_t*>((reinterpret_cast<uintptr_t>(p) + 255) & ~uintptr_t(255));
  T* r = reinterpret_cast<T*>(p);
  p += sizeof(T) * count;
  return r;
}

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

}  // namespace

struct cbd_ctx {
  cbd_model_config cfg{};
  cbd_limits lim{};
  int fmt = FMT_BF16;
  int kv_bits = 0;  // affine slabs: 8- or 4-bit codes (0: bf16 slabs)
  int q_dim = 0, kv_dim = 0, qkv_dim = 0;
  const uint16_t* embed = nullptr;
  const uint16_t* final_norm = nullptr;
  Mat lm_head{};
  std::vector<LayerW> layers;

  uint8_t* arena = nullptr;
  size_t arena_bytes = 0;
  int64_t granule_bytes = 0;
  int64_t n_granules = 0;
  std::map<int64_t, int64_t> free_runs;  // first granule -> run length
  std::vector<Slab> slabs;
  cbd_stats_t stats{};

  bool host_only = true;
  int rows_pad = 0;  // activation rows available (multiple of 128)
  void* ws = nullptr;
  float* h = nullptr;       // residual stream fp32 [R, d]
  uint16_t* xa = nullptr;   // planes of gain * h for the next norm's consumer [2][R, d]
  uint16_t* xo = nullptr;   // planes of the attention output [2][R, q_dim]
  uint16_t* xm = nullptr;   // planes of the SwiGLU product [2][R, max(F, d)]
  float* ss = nullptr;      // per-16-feature sums of squares of h [d/16][R]
  float* ss_head = nullptr; // the same for the rows gathered for a prefill's lm_head [d/16][64]
  float* gemm_part = nullptr;   // split-K partial tiles
  int32_t* gemm_counters = nullptr;  // split-K arrival counters, one per row block
  int32_t* attn_counters = nullptr;  // split-attention arrival counters [64][n_kv_heads]
  float* argmax_part = nullptr;      // argmax (max, index) pairs [64][kArgmaxSegments]
  int32_t* argmax_counters = nullptr;  // argmax arrival counters [64]
  SampleWs sample_ws{};                // sampling workspace (weights, chunk histograms, row state)
  size_t gemm_part_bytes = 0;
  int gemm_counter_count = 0;
  float* qkv = nullptr;
  int64_t xa_plane = 0, xo_plane = 0, xm_plane = 0;
  float* part_o = nullptr;
  float* part_ml = nullptr;
  float* rope_cs = nullptr;
  uint8_t* meta_dev = nullptr;  // device copy of one staging slot
  size_t slot_bytes = 0;
  uint8_t* staging = nullptr;   // pinned host, kStagingSlots slots
  hipEvent_t slot_ev[kStagingSlots] = {};
  int next_slot = 0;

  // per-kernel event timing (cbd_profile_begin / cbd_profile_end)
  uint32_t prof_mask = 0;
  int prof_max = 0;
  int prof_every = 1;      // time one selected launch in prof_every
  int64_t prof_seen = 0;   // selected launches so far
  std::vector<hipEvent_t> prof_ev;  // 2 per recorded launch
  struct ProfRec {
    int kind;
    double bytes, flops;
  };
  std::vector<ProfRec> prof_rec;
};

// ----------------------------------------------------------------------------- metadata staging

namespace {

struct MetaLayout {
  size_t meta_off, items_off, parts_off, idx_off, total;
};

MetaLayout meta_layout(const cbd_ctx* c) {
  MetaLayout m;
  const size_t rows = (size_t)c->rows_pad;
  m.meta_off = 0;
  m.items_off = round_up(m.meta_off + rows * sizeof(RowMeta), 256);
  m.parts_off = round_up(m.items_off + (rows + kExtraItems) * sizeof(AttnItem), 256);
  m.idx_off = round_up(m.parts_off + rows * sizeof(int32_t) * 2, 256);
  m.total = round_up(m.idx_off + 64 * sizeof(int32_t), 256);
  return m;
}

// Reserve a pinned staging slot whose previous upload has completed.
uint8_t* staging_slot(cbd_ctx* c, int* slot_out) {
  const int s = c->next_slot;
  c->next_slot = (c->next_slot + 1) % kStagingSlots;
  (void)hipEventSynchronize(c->slot_ev[s]);
  *slot_out = s;
  return c->staging + (size_t)s * c->slot_bytes;
}

cbd_status upload(cbd_ctx* c, int slot, size_t bytes, hipStream_t st) {
  HIP_TRY(hipMemcpyAsync(c->meta_dev, c->staging + (size_t)slot * c->slot_bytes, bytes, hipMemcpyHostToDevice, st),
          "metadata upload");
  HIP_TRY(hipEventRecord(c->slot_ev[slot], st), "event record");
  return CBD_OK;
}

bool valid_model(const cbd_model_config* m, std::string* why) {
  char buf[256];
  auto bad = [&](const char* s) { *why = s; return false; };
  if (m->n_layers < 1 || m->d_model < 1 || m->n_heads < 1 || m->n_kv_heads < 1 || m->ffn_dim < 1 || m->vocab < 1)
    return bad("model sizes must be positive");
  if (m->head_dim != 64 && m->head_dim != 128) return bad("head_dim must be 64 or 128");
  if (m->n_heads % m->n_kv_heads) return bad("n_heads must be a multiple of n_kv_heads");
  const int G = m->n_heads / m->n_kv_heads;
  if (G != 1 && G != 2 && G != 4) return bad("n_heads / n_kv_heads must be 1, 2 or 4");
  const int kmul = m->weight_format == CBD_WEIGHTS_INT4 ? 512 : 256;
  if (m->weight_format != CBD_WEIGHTS_BF16 && m->weight_format != CBD_WEIGHTS_INT4) return bad("unknown weight_format");
  if (m->d_model % kmul || m->ffn_dim % kmul || (m->n_heads * m->head_dim) % kmul) {
    snprintf(buf, sizeof buf, "d_model, ffn_dim and n_heads*head_dim must be multiples of %d", kmul);
    return bad(buf);
  }
  if (m->vocab % 64 || (m->n_kv_heads * m->head_dim) % 64) return bad("vocab and kv width must be multiples of 64");
  if (m->max_position < 1) return bad("max_position must be positive");
  if (m->kv_format != CBD_KV_BF16 && m->kv_format != CBD_KV_AFFINE8 && m->kv_format != CBD_KV_AFFINE4)
    return bad("unknown kv_format");
  if (!(m->rms_eps >= 0.f) || !(m->rope_theta > 0.f)) return bad("rms_eps >= 0 and rope_theta > 0 required");
  return true;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Build the (row, key range) work items of one decode step. The attention kernel runs one wave per
// item and KV head and streams keys in blocks of 32, so ranges start at multiples of 32. Ranges are
// sized so that about kDecodeWaves waves cover the step's keys, at least kMinChunk keys each; every
// split of a row gets a partial slot. Steps of at most kFewRows rows over bf16 or 8-bit K/V aim at
// kDecodeWavesFew waves (one per SIMD): a wave with two bf16 blocks in flight streams about 13 GB/s,
// so about 600 waves already reach the HBM rate, and more waves only add splits that the merges pay
// for (32k-token rows: 188 -> 170 us per layer). Larger batches (each row needs few splits; more waves
// even out the tail) and 4-bit K/V (a fifth of the bytes per key: more waves to reach the rate) keep
// two per SIMD.
#ifndef CBD_DECODE_WAVES
#define CBD_DECODE_WAVES 2048
#endif
#ifndef CBD_DECODE_WAVES_FEW
#define CBD_DECODE_WAVES_FEW 1024
#endif
constexpr size_t kFewRows = 16;
#ifndef CBD_DECODE_MERGE_CAP
#define CBD_DECODE_MERGE_CAP 1
#endif
constexpr int64_t kMergeBatch = 8;  // splits whose partials the merging wave loads in one round trip
constexpr int64_t kMergeCapMinWaves = 384;
#ifndef CBD_DECODE_MIN_CHUNK
#define CBD_DECODE_MIN_CHUNK 256
#endif
constexpr int64_t kDecodeWaves = CBD_DECODE_WAVES, kDecodeWavesFew = CBD_DECODE_WAVES_FEW;
constexpr int64_t kMinChunk = CBD_DECODE_MIN_CHUNK;
constexpr int64_t kMaxSplits = 64;
int plan_decode_items(const cbd_ctx* c, const std::vector<RowMeta>& rows, AttnItem* items, int32_t* row_parts) {
  int64_t total = 0;
  for (const RowMeta& r : rows) total += r.pos + 1;
  const bool few = rows.size() <= kFewRows && c->cfg.kv_format != CBD_KV_AFFINE4;
  const int64_t waves = few ? kDecodeWavesFew : kDecodeWaves;
  const int64_t per_wave = (total * c->cfg.n_kv_heads + waves - 1) / waves;
  int64_t longest = 0;
  bool forked = false;
  for (const RowMeta& r : rows) {
    longest = std::max<int64_t>(longest, r.pos + 1);
    forked |= r.pre_end > 0;
  }
  // at most kMaxSplits splits per row: the merge reads one (max, sum) pair per lane (a fork's range
  // is cut at its prefix boundary too, which can add one split)
  int64_t max_splits = forked ? kMaxSplits - 1 : kMaxSplits;
  // Few-row steps over bf16 K/V also keep each row within one merge round trip (kMergeBatch
  // splits) where the longer ranges still give at least kMergeCapMinWaves waves: Mistral-7B int4
  // step (contexts 1k..8k) 2544 -> 2659 tok/s, B = 16 +2.8%, 32k-token rows +1%; B = 4 (too few
  // waves left) -3% and 8-bit K/V (a wave streams codes more slowly) -24% keep the longer split list.
  if (few && CBD_DECODE_MERGE_CAP && c->cfg.kv_format == CBD_KV_BF16) {
    const int64_t cap = forked ? kMergeBatch - 1 : kMergeBatch;
    const int64_t cap_chunk = round_up((longest + cap - 1) / cap, 32);
    if (total * c->cfg.n_kv_heads / std::max<int64_t>(cap_chunk, kMinChunk) >= kMergeCapMinWaves) max_splits = cap;
  }
  int64_t chunk = std::max({kMinChunk, round_up(per_wave, 32), round_up((longest + max_splits - 1) / max_splits, 32)});
  for (;;) {
    int64_t slots = 0;
    for (const RowMeta& r : rows) {
      const int64_t s = (r.pre_end + chunk - 1) / chunk + (r.pos + 1 - r.pre_end + chunk - 1) / chunk;
      if (s > 1) slots += s;
    }
    if (slots <= kMaxParts) break;
    chunk *= 2;
  }
  int n = 0, slot = 0;
  for (size_t i = 0; i < rows.size(); ++i) {
    const RowMeta& r = rows[i];
    const int nk = r.pos + 1;
    // a fork's keys below pre_end are items over the parent's slab, the rest over its own
    const int pre = r.pre_end;
    const int pre_splits = (int)((pre + chunk - 1) / chunk);
    const int splits = pre_splits + (int)((nk - pre + chunk - 1) / chunk);
    if (splits <= 1) {
      items[n++] = AttnItem{r.slab_off, r.stride, r.pos, (int32_t)i, 0, nk, -1, 0, 0, 0};
      row_parts[2 * i] = 0;
      row_parts[2 * i + 1] = 0;
    } else {
      row_parts[2 * i] = slot;
      row_parts[2 * i + 1] = splits;
      for (int s = 0; s < pre_splits; ++s) {
        const int b = (int)(s * chunk), e = (int)std::min<int64_t>(pre, (s + 1) * chunk);
        items[n++] = AttnItem{r.pre_off, r.pre_stride, r.pos, (int32_t)i, b, e, slot++, 0, 0, 0};
      }
      for (int s = 0; s < splits - pre_splits; ++s) {
        const int b = pre + (int)(s * chunk), e = (int)std::min<int64_t>(nk, pre + (s + 1) * chunk);
        items[n++] = AttnItem{r.slab_off, r.stride, r.pos, (int32_t)i, b, e, slot++, 0, 0, 0};
      }
    }
  }
  return n;
}

}  // namespace

namespace cbd {
cbd_status record_error(cbd_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

LaunchEvents& launch_events() {
  static thread_local LaunchEvents ev{nullptr, nullptr};
  return ev;
}
}  // namespace cbd

namespace {

// Time the first kernel launched inside the scope when its kind is being profiled: the launch
// helper stamps the pair of events at that kernel's own start and end.
struct ProfScope {
  cbd_ctx* c;
  hipStream_t st;
  bool on;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  ProfScope(cbd_ctx* c_, int kind, double bytes, double flops, hipStream_t st_) : c(c_), st(st_), on(false) {
    if (!(c->prof_mask & (1u << kind)) || (int)c->prof_rec.size() >= c->prof_max) return;
    if (c->prof_seen++ % c->prof_every) return;
    const size_t i = c->prof_rec.size();
    c->prof_rec.push_back({kind, bytes, flops});
    e0 = c->prof_ev[2 * i];
    e1 = c->prof_ev[2 * i + 1];
    cbd::launch_events() = cbd::LaunchEvents{e0, e1};
    on = true;
  }
  ~ProfScope() {
    if (!on) return;
    cbd::LaunchEvents& ev = cbd::launch_events();
    if (ev.start == e0) {  // nothing was launched (or the launch was refused): record an empty interval
      ev = cbd::LaunchEvents{nullptr, nullptr};
      (void)hipEventRecord(e0, st);
      (void)hipEventRecord(e1, st);
    }
  }
};

}  // namespace

// ----------------------------------------------------------------------------- create / destroy

extern "C" size_t cbd_kv_bytes_per_token(const cbd_model_config* cfg) {
  if (!cfg) return 0;
  if (cfg->kv_format == CBD_KV_AFFINE8 || cfg->kv_format == CBD_KV_AFFINE4)
    return (size_t)cfg->n_layers * 2 * cfg->n_kv_heads *
           (cfg->head_dim * (cfg->kv_format == CBD_KV_AFFINE8 ? 8 : 4) / 8 + cfg->head_dim / kQGroup * 8);
  return (size_t)cfg->n_layers * 2 * cfg->n_kv_heads * cfg->head_dim * 2;
}

extern "C" int32_t cbd_slab_granule_tokens(void) { return kGranuleTokens; }

extern "C" const char* cbd_last_error(void) { return g_err.c_str(); }

static cbd_status setup_weights(cbd_ctx* c, const cbd_weights* w) {
  auto mat = [&](const cbd_matrix& m, const char* name, Mat* out) -> cbd_status {
    if (!m.data || !aligned16(m.data)) return fail(CBD_E_INVAL, "weight %s: null or not 16-byte aligned", name);
    if (c->fmt == FMT_INT4 && (!m.aux || !aligned16(m.aux)))
      return fail(CBD_E_INVAL, "weight %s: int4 scale/bias pairs missing or misaligned", name);
    *out = Mat{m.data, m.aux};
    return CBD_OK;
  };
  auto vec = [&](const void* p, const char* name, const uint16_t** out) -> cbd_status {
    if (!p || !aligned16(p)) return fail(CBD_E_INVAL, "%s: null or not 16-byte aligned", name);
    *out = static_cast<const uint16_t*>(p);
    return CBD_OK;
  };
  cbd_status s;
  if (!w || !w->layers) return fail(CBD_E_INVAL, "weights missing");
  if ((s = vec(w->embed, "embed", &c->embed))) return s;
  if ((s = vec(w->final_norm, "final_norm", &c->final_norm))) return s;
  if ((s = mat(w->lm_head, "lm_head", &c->lm_head))) return s;
  c->layers.resize(c->cfg.n_layers);
  for (int l = 0; l < c->cfg.n_layers; ++l) {
    const cbd_layer_weights& L = w->layers[l];
    LayerW& o = c->layers[l];
    if ((s = vec(L.attn_norm, "attn_norm", &o.attn_norm)) || (s = vec(L.ffn_norm, "ffn_norm", &o.ffn_norm)) ||
        (s = mat(L.wq, "wq", &o.wq)) || (s = mat(L.wk, "wk", &o.wk)) || (s = mat(L.wv, "wv", &o.wv)) ||
        (s = mat(L.wo, "wo", &o.wo)) || (s = mat(L.w_gate, "w_gate", &o.wg)) || (s = mat(L.w_up, "w_up", &o.wu)) ||
        (s = mat(L.w_down, "w_down", &o.wd)))
      return s;
  }
  return CBD_OK;
}

static cbd_status setup_device(cbd_ctx* c) {
  const cbd_model_config& m = c->cfg;
  {  // the products even their work out over the device's compute units
    int dev = 0, units = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&units, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
      set_plan_compute_units(units);
  }
  const int rows = std::max(c->lim.max_batch, c->lim.max_prefill_tokens);
  c->rows_pad = (int)round_up(std::max(rows, 128), 128);  // whole 128-row tiles of the dense product
  const size_t R = (size_t)c->rows_pad;
  const size_t G = (size_t)m.n_heads;
  const size_t half = (size_t)m.head_dim / 2;
  const MetaLayout ml = meta_layout(c);
  c->slot_bytes = ml.total;
  size_t bytes = 0;
  const size_t wm = std::max(m.ffn_dim, m.d_model);
  // split-K workspace: the largest any decode-size launch plans (cbd_linear included)
  {
    const int shapes[][3] = {{EPI_STORE, c->qkv_dim, m.d_model},  {EPI_RESIDUAL, m.d_model, c->q_dim},
                             {EPI_SWIGLU, m.ffn_dim, m.d_model},  {EPI_RESIDUAL, m.d_model, m.ffn_dim},
                             {EPI_STORE, m.vocab, m.d_model}};
    for (int rows = 1; rows <= 64; ++rows)
      for (const auto& sh : shapes) {
        const SkinnyPlan pl = plan_skinny(sh[0], c->fmt, sh[1], sh[2], rows, 1, 0);
        c->gemm_part_bytes = std::max(c->gemm_part_bytes, skinny_part_bytes(pl));
        c->gemm_counter_count = std::max(c->gemm_counter_count, pl.row_blocks);
      }
    c->gemm_part_bytes = std::max<size_t>(c->gemm_part_bytes, 64u << 20);  // room for cbd_linear plans
    c->gemm_counter_count = std::max(c->gemm_counter_count, 1 << 16);
  }
  bytes += c->gemm_part_bytes + 256;
  bytes += (size_t)c->gemm_counter_count * 4 + 256;
  bytes += (size_t)64 * m.n_kv_heads * 4 + 256;
  bytes += (size_t)64 * kArgmaxSegments * 2 * 4 + 256 + 64 * 4 + 256;  // argmax pairs and counters
  bytes += R * m.d_model * 4 + 256;                 // h
  bytes += 2 * R * m.d_model * 2 + 256;             // xa planes
  bytes += 2 * R * c->q_dim * 2 + 256;              // xo planes
  bytes += 2 * R * wm * 2 + 256;                    // xm planes (also the standalone-linear input)
  bytes += (size_t)(m.d_model / 16) * R * 4 + 256;  // ss
  bytes += (size_t)(m.d_model / 16) * 64 * 4 + 256;  // ss_head
  bytes += R * c->qkv_dim * 4 + 256;                // qkv
  bytes += (size_t)kMaxParts * G * m.head_dim * 4 + 256;  // partial outputs
  bytes += (size_t)kMaxParts * G * 2 * 4 + 256;     // partial (max, sum)
  bytes += (size_t)m.max_position * half * 2 * 4 + 256;  // rope table
  bytes += ml.total + 256;                          // metadata
  const size_t sample_bytes = sample_ws_layout(nullptr, m.vocab).bytes;
  bytes += sample_bytes + 256;                      // sampling workspace
  HIP_TRY(hipMalloc(&c->ws, bytes), "workspace allocation");
  HIP_TRY(hipMemset(c->ws, 0, bytes), "workspace clear");
  uint8_t* p = static_cast<uint8_t*>(c->ws);
  c->h = align_ptr<float>(p, R * m.d_model);
  c->xa = align_ptr<uint16_t>(p, 2 * R * m.d_model);
  c->xo = align_ptr<uint16_t>(p, 2 * R * c->q_dim);
  c->xm = align_ptr<uint16_t>(p, 2 * R * wm);
  c->ss = align_ptr<float>(p, (size_t)(m.d_model / 16) * R);
  c->ss_head = align_ptr<float>(p, (size_t)(m.d_model / 16) * 64);
  c->gemm_part = align_ptr<float>(p, c->gemm_part_bytes / 4);
  c->gemm_counters = align_ptr<int32_t>(p, c->gemm_counter_count);
  c->attn_counters = align_ptr<int32_t>(p, (size_t)64 * m.n_kv_heads);
  c->argmax_part = align_ptr<float>(p, (size_t)64 * kArgmaxSegments * 2);
  c->argmax_counters = align_ptr<int32_t>(p, 64);
  c->qkv = align_ptr<float>(p, R * c->qkv_dim);
  // the lo value of an activation pair sits kXLo elements after its hi value (common.h)
  c->xa_plane = kXLo;
  c->xo_plane = kXLo;
  c->xm_plane = kXLo;
  c->part_o = align_ptr<float>(p, (size_t)kMaxParts * G * m.head_dim);
  c->part_ml = align_ptr<float>(p, (size_t)kMaxParts * G * 2);
  c->rope_cs = align_ptr<float>(p, (size_t)m.max_position * half * 2);
  c->meta_dev = align_ptr<uint8_t>(p, ml.total);
  c->sample_ws = sample_ws_layout(align_ptr<uint8_t>(p, sample_bytes), m.vocab);

  // RoPE table: angles in double precision, stored as fp32 (cos, sin) pairs
  std::vector<float> cs((size_t)m.max_position * half * 2);
  for (int t = 0; t < m.max_position; ++t)
    for (size_t i = 0; i < half; ++i) {
      const double inv_freq = std::pow((double)m.rope_theta, -2.0 * (double)i / (double)m.head_dim);
      const double a = (double)t * inv_freq;
      cs[((size_t)t * half + i) * 2 + 0] = (float)std::cos(a);
      cs[((size_t)t * half + i) * 2 + 1] = (float)std::sin(a);
    }
  HIP_TRY(hipMemcpy(c->rope_cs, cs.data(), cs.size() * 4, hipMemcpyHostToDevice), "rope table upload");
  HIP_TRY(hipHostMalloc(reinterpret_cast<void**>(&c->staging), c->slot_bytes * kStagingSlots, hipHostMallocDefault),
          "pinned staging allocation");
  for (int i = 0; i < kStagingSlots; ++i)
    HIP_TRY(hipEventCreateWithFlags(&c->slot_ev[i], hipEventDisableTiming), "event create");
  return CBD_OK;
}

static void release(cbd_ctx* c) {
  if (!c) return;
  if (!c->host_only) {
    (void)hipDeviceSynchronize();
    for (hipEvent_t e : c->prof_ev) (void)hipEventDestroy(e);
    for (int i = 0; i < kStagingSlots; ++i)
      if (c->slot_ev[i]) (void)hipEventDestroy(c->slot_ev[i]);
    if (c->staging) (void)hipHostFree(c->staging);
    if (c->ws) (void)hipFree(c->ws);
  }
  delete c;
}

extern "C" cbd_status cbd_create(const cbd_model_config* cfg, const cbd_weights* weights, const cbd_limits* limits,
                                 void* kv_arena_dev, size_t arena_bytes, cbd_ctx** out) {
  if (!cfg || !limits || !out) return fail(CBD_E_INVAL, "cbd_create: null argument");
  *out = nullptr;
  std::string why;
  if (!valid_model(cfg, &why)) return fail(CBD_E_INVAL, "cbd_create: %s", why.c_str());
  if (limits->max_batch < 1 || limits->max_batch > 64) return fail(CBD_E_INVAL, "max_batch must be in 1..64");
  if (limits->max_segments < 1 || limits->max_segments > 64) return fail(CBD_E_INVAL, "max_segments must be in 1..64");
  if (limits->max_prefill_tokens < 1 || limits->max_prefill_tokens > (1 << 20))
    return fail(CBD_E_INVAL, "max_prefill_tokens must be in 1..2^20");
  cbd_ctx* c = new cbd_ctx();
  c->cfg = *cfg;
  c->lim = *limits;
  c->host_only = limits->host_only != 0;
  c->fmt = cfg->weight_format == CBD_WEIGHTS_INT4 ? FMT_INT4 : FMT_BF16;
  c->kv_bits = cfg->kv_format == CBD_KV_AFFINE8 ? 8 : cfg->kv_format == CBD_KV_AFFINE4 ? 4 : 0;
  c->q_dim = cfg->n_heads * cfg->head_dim;
  c->kv_dim = cfg->n_kv_heads * cfg->head_dim;
  c->qkv_dim = c->q_dim + 2 * c->kv_dim;
  c->arena = static_cast<uint8_t*>(kv_arena_dev);
  c->arena_bytes = arena_bytes;
  c->granule_bytes = (int64_t)kGranuleTokens * (int64_t)cbd_kv_bytes_per_token(cfg);
  c->n_granules = (int64_t)(arena_bytes / (size_t)c->granule_bytes);
  if (c->n_granules > 0) c->free_runs[0] = c->n_granules;
  c->stats.arena_bytes = (int64_t)arena_bytes;
  cbd_status s = CBD_OK;
  if (!c->host_only) {
    if (!kv_arena_dev || (reinterpret_cast<uintptr_t>(kv_arena_dev) & 255)) {
      s = fail(CBD_E_INVAL, "kv arena must be a 256-byte aligned device pointer");
    } else if ((s = setup_weights(c, weights)) == CBD_OK && (s = setup_device(c)) == CBD_OK) {
      // masked keys get probability 0, and 0 x (finite V) = 0: the arena starts cleared so that the
      // slab positions beyond a sequence's length never hold non-finite bit patterns
      if (hipMemset(kv_arena_dev, 0, arena_bytes) != hipSuccess || hipDeviceSynchronize() != hipSuccess)
        s = fail(CBD_E_HIP, "kv arena clear failed");
    }
  }
  if (s != CBD_OK) {
    release(c);
    return s;
  }
  *out = c;
  return CBD_OK;
}

extern "C" cbd_status cbd_destroy(cbd_ctx* ctx) {
  if (!ctx) return fail(CBD_E_INVAL, "cbd_destroy: null context");
  release(ctx);
  return CBD_OK;
}

extern "C" cbd_status cbd_stats(const cbd_ctx* ctx, cbd_stats_t* out) {
  if (!ctx || !out) return fail(CBD_E_INVAL, "cbd_stats: null argument");
  *out = ctx->stats;
  return CBD_OK;
}

// ----------------------------------------------------------------------------- slabs

static cbd_status live_slab(const cbd_ctx* c, int32_t id, const Slab** out) {
  if (id < 0 || (size_t)id >= c->slabs.size() || !c->slabs[id].live)
    return fail(CBD_E_BADSEQ, "sequence id %d is not live", id);
  *out = &c->slabs[id];
  return CBD_OK;
}

// Take a first-fit run of `need` granules (CBD_E_NOSPACE when none is free).
static cbd_status take_granules(cbd_ctx* c, int64_t need, int64_t* first_out, const char* who) {
  if (need > c->n_granules)
    return fail(CBD_E_CAPACITY, "%s: %lld granules exceed the whole arena (%lld)", who, (long long)need,
                (long long)c->n_granules);
  auto it = c->free_runs.begin();
  for (; it != c->free_runs.end(); ++it)
    if (it->second >= need) break;
  if (it == c->free_runs.end()) return fail(CBD_E_NOSPACE, "%s: no free run of %lld granules", who, (long long)need);
  const int64_t first = it->first, run = it->second;
  c->free_runs.erase(it);
  if (run > need) c->free_runs[first + need] = run - need;
  c->stats.arena_bytes_used += need * c->granule_bytes;
  *first_out = first;
  return CBD_OK;
}

static void give_granules(cbd_ctx* c, int64_t first, int64_t count) {
  c->stats.arena_bytes_used -= count * c->granule_bytes;
  auto next = c->free_runs.lower_bound(first);
  if (next != c->free_runs.end() && next->first == first + count) {
    count += next->second;
    c->free_runs.erase(next);
  }
  auto prev = c->free_runs.lower_bound(first);
  if (prev != c->free_runs.begin()) {
    --prev;
    if (prev->first + prev->second == first) {
      first = prev->first;
      count += prev->second;
      c->free_runs.erase(prev);
    }
  }
  c->free_runs[first] = count;
}

// A new live slab record over granules [first, first + need), its own keys starting at base.
static int32_t new_slab(cbd_ctx* c, int64_t first, int64_t need, int32_t base) {
  int32_t id = 0;
  while ((size_t)id < c->slabs.size() && (c->slabs[id].live || c->slabs[id].zombie)) ++id;
  if ((size_t)id == c->slabs.size()) c->slabs.emplace_back();
  Slab& s = c->slabs[id];
  s = Slab{};
  s.live = true;
  s.base = base;
  s.cap = (int32_t)std::min<int64_t>(base + need * kGranuleTokens, c->cfg.max_position);
  s.stride = (int32_t)(need * kGranuleTokens);
  s.gran_begin = first;
  s.gran_count = need;
  s.off = first * c->granule_bytes;
  c->stats.live_seqs += 1;
  return id;
}

extern "C" cbd_status kvslab_alloc(cbd_ctx* c, int32_t capacity_tokens, int32_t* seq_id_out) {
  if (!c || !seq_id_out) return fail(CBD_E_INVAL, "kvslab_alloc: null argument");
  if (capacity_tokens < 1) return fail(CBD_E_INVAL, "kvslab_alloc: capacity must be >= 1");
  if (capacity_tokens > c->cfg.max_position)
    return fail(CBD_E_CAPACITY, "kvslab_alloc: capacity %d exceeds max_position %d", capacity_tokens,
                c->cfg.max_position);
  const int64_t need = (capacity_tokens + kGranuleTokens - 1) / kGranuleTokens;
  int64_t first;
  if (cbd_status st = take_granules(c, need, &first, "kvslab_alloc")) return st;
  *seq_id_out = new_slab(c, first, need, 0);
  return CBD_OK;
}

// Bytes of one block of 32 keys in one (layer, K or V, KV head) region, and of a whole region.
static int64_t kv_block_bytes(const cbd_ctx* c) {
  return c->kv_bits ? q_block_bytes(c->cfg.head_dim, c->kv_bits) : (int64_t)32 * c->cfg.head_dim * 2;
}
static int64_t kv_region_bytes(const cbd_ctx* c, int32_t stride) { return (int64_t)(stride / 32) * kv_block_bytes(c); }

// The kernels' view of a slab at position pos: own keys addressed from a slab_off shifted back by
// base / 32 blocks, keys below base in the parent's slab.
static RowMeta row_meta(const cbd_ctx* c, const Slab& s, int32_t pos) {
  RowMeta m{s.off - (int64_t)(s.base / 32) * kv_block_bytes(c), s.stride, pos, 0, 0, 0};
  if (s.parent >= 0) {
    const Slab& p = c->slabs[s.parent];
    m.pre_off = p.off;
    m.pre_stride = p.stride;
    m.pre_end = s.base;
  }
  return m;
}

extern "C" cbd_status kvslab_fork(cbd_ctx* c, int32_t parent_id, int32_t prefix_len, int32_t capacity_tokens,
                                  int32_t* seq_id_out, cbd_stream stream) {
  if (!c || !seq_id_out) return fail(CBD_E_INVAL, "kvslab_fork: null argument");
  const Slab* pp;
  if (cbd_status st = live_slab(c, parent_id, &pp)) return st;
  if (pp->parent >= 0) return fail(CBD_E_INVAL, "kvslab_fork: sequence %d is itself a fork", parent_id);
  if (prefix_len < 0 || prefix_len > pp->len)
    return fail(CBD_E_INVAL, "kvslab_fork: prefix %d outside the parent's %d tokens", prefix_len, pp->len);
  if (capacity_tokens <= prefix_len)
    return fail(CBD_E_INVAL, "kvslab_fork: capacity %d leaves no room after the prefix %d", capacity_tokens, prefix_len);
  if (capacity_tokens > c->cfg.max_position)
    return fail(CBD_E_CAPACITY, "kvslab_fork: capacity %d exceeds max_position %d", capacity_tokens,
                c->cfg.max_position);
  const int32_t base = prefix_len / 32 * 32;  // whole blocks stay shared
  const int64_t need = (capacity_tokens - base + kGranuleTokens - 1) / kGranuleTokens;
  int64_t first;
  if (cbd_status st = take_granules(c, need, &first, "kvslab_fork")) return st;
  const int32_t id = new_slab(c, first, need, base);
  Slab& s = c->slabs[id];
  Slab& p = c->slabs[parent_id];
  s.parent = parent_id;
  s.len = prefix_len;
  p.children += 1;
  if (prefix_len > base && !c->host_only) {
    // the block holding the prefix's last keys is copied (its later keys are the fork's own)
    const int64_t bb = kv_block_bytes(c);
    const int64_t rows = (int64_t)c->cfg.n_layers * 2 * c->cfg.n_kv_heads;
    HIP_TRY(hipMemcpy2DAsync(c->arena + s.off, (size_t)kv_region_bytes(c, s.stride),
                             c->arena + p.off + (int64_t)(base / 32) * bb, (size_t)kv_region_bytes(c, p.stride),
                             (size_t)bb, (size_t)rows, hipMemcpyDeviceToDevice, static_cast<hipStream_t>(stream)),
            "kvslab_fork boundary block copy");
  }
  *seq_id_out = id;
  return CBD_OK;
}

extern "C" cbd_status kvslab_free(cbd_ctx* c, int32_t seq_id) {
  if (!c) return fail(CBD_E_INVAL, "kvslab_free: null context");
  const Slab* sp;
  if (cbd_status st = live_slab(c, seq_id, &sp)) return st;
  Slab& s = c->slabs[seq_id];
  c->stats.live_seqs -= 1;
  if (s.children > 0) {  // forks still read its prefix: keep the granules until the last one goes
    s.live = false;
    s.zombie = true;
    return CBD_OK;
  }
  give_granules(c, s.gran_begin, s.gran_count);
  const int32_t parent = s.parent;
  s = Slab{};
  if (parent >= 0) {
    Slab& p = c->slabs[parent];
    p.children -= 1;
    if (p.zombie && p.children == 0) {
      give_granules(c, p.gran_begin, p.gran_count);
      p = Slab{};
    }
  }
  return CBD_OK;
}

extern "C" cbd_status kvslab_len(const cbd_ctx* c, int32_t seq_id, int32_t* len_out) {
  if (!c || !len_out) return fail(CBD_E_INVAL, "kvslab_len: null argument");
  const Slab* s;
  if (cbd_status st = live_slab(c, seq_id, &s)) return st;
  *len_out = s->len;
  return CBD_OK;
}

extern "C" cbd_status kvslab_capacity(const cbd_ctx* c, int32_t seq_id, int32_t* cap_out) {
  if (!c || !cap_out) return fail(CBD_E_INVAL, "kvslab_capacity: null argument");
  const Slab* s;
  if (cbd_status st = live_slab(c, seq_id, &s)) return st;
  *cap_out = s->cap;
  return CBD_OK;
}

extern "C" cbd_status kvslab_append(cbd_ctx* c, int32_t seq_id, int32_t n_tokens, const void* k_dev,
                                    const void* v_dev, cbd_stream stream) {
  if (!c) return fail(CBD_E_INVAL, "kvslab_append: null context");
  const Slab* s;
  if (cbd_status st = live_slab(c, seq_id, &s)) return st;
  if (n_tokens < 0) return fail(CBD_E_INVAL, "kvslab_append: negative count");
  if ((int64_t)s->len + n_tokens > s->cap)
    return fail(CBD_E_CAPACITY, "kvslab_append: %d + %d exceeds capacity %d", s->len, n_tokens, s->cap);
  if (n_tokens == 0) return CBD_OK;
  if (!k_dev || !v_dev || !aligned16(k_dev) || !aligned16(v_dev))
    return fail(CBD_E_INVAL, "kvslab_append: K/V must be 16-byte aligned device pointers");
  if (c->host_only) return fail(CBD_E_NODEVICE, "kvslab_append: host-only context");
  const int64_t off = row_meta(c, *s, s->len).slab_off;  // positions >= len >= base: the own part
  if (c->kv_bits)
    HIP_TRY(launch_slab_q8(c->arena, off, s->stride, s->len, n_tokens, n_tokens, 0, c->cfg.n_layers,
                           c->cfg.n_kv_heads, c->cfg.head_dim, static_cast<const uint16_t*>(k_dev),
                           static_cast<const uint16_t*>(v_dev), nullptr, nullptr, c->kv_bits,
                           static_cast<hipStream_t>(stream)),
            "kvslab_append launch");
  else
    HIP_TRY(launch_slab_copy(c->arena, off, s->stride, s->len, n_tokens, n_tokens, 0, c->cfg.n_layers,
                             c->cfg.n_kv_heads, c->cfg.head_dim, static_cast<const uint16_t*>(k_dev),
                             static_cast<const uint16_t*>(v_dev), nullptr, nullptr, static_cast<hipStream_t>(stream)),
            "kvslab_append launch");
  c->slabs[seq_id].len += n_tokens;
  return CBD_OK;
}

extern "C" cbd_status kvslab_read(const cbd_ctx* c, int32_t seq_id, int32_t start, int32_t n_tokens, void* k_out_dev,
                                  void* v_out_dev, cbd_stream stream) {
  if (!c) return fail(CBD_E_INVAL, "kvslab_read: null context");
  if (c->kv_bits) return fail(CBD_E_UNSUPPORTED, "kvslab_read: affine slabs are read with kvslab_read_q8");
  const Slab* s;
  if (cbd_status st = live_slab(c, seq_id, &s)) return st;
  if (start < 0 || n_tokens < 0) return fail(CBD_E_INVAL, "kvslab_read: negative range");
  if ((int64_t)start + n_tokens > s->len)
    return fail(CBD_E_CAPACITY, "kvslab_read: [%d, %d) beyond length %d", start, start + n_tokens, s->len);
  if (n_tokens == 0) return CBD_OK;
  if (!k_out_dev || !v_out_dev || !aligned16(k_out_dev) || !aligned16(v_out_dev))
    return fail(CBD_E_INVAL, "kvslab_read: outputs must be 16-byte aligned device pointers");
  if (c->host_only) return fail(CBD_E_NODEVICE, "kvslab_read: host-only context");
  // a fork's positions below its base are read from the parent's slab
  const RowMeta m = row_meta(c, *s, start);
  const int32_t end = start + n_tokens, cut = std::min(std::max(start, m.pre_end), end);
  if (cut > start)
    HIP_TRY(launch_slab_copy(c->arena, m.pre_off, m.pre_stride, start, cut - start, n_tokens, 0, c->cfg.n_layers,
                             c->cfg.n_kv_heads, c->cfg.head_dim, nullptr, nullptr, static_cast<uint16_t*>(k_out_dev),
                             static_cast<uint16_t*>(v_out_dev), static_cast<hipStream_t>(stream)),
            "kvslab_read launch");
  if (end > cut)
    HIP_TRY(launch_slab_copy(c->arena, m.slab_off, s->stride, cut, end - cut, n_tokens, cut - start, c->cfg.n_layers,
                             c->cfg.n_kv_heads, c->cfg.head_dim, nullptr, nullptr, static_cast<uint16_t*>(k_out_dev),
                             static_cast<uint16_t*>(v_out_dev), static_cast<hipStream_t>(stream)),
            "kvslab_read launch");
  return CBD_OK;
}

extern "C" cbd_status kvslab_read_q8(const cbd_ctx* c, int32_t seq_id, int32_t start, int32_t n_tokens,
                                     void* codes_out_dev, void* sb_out_dev, cbd_stream stream) {
  if (!c) return fail(CBD_E_INVAL, "kvslab_read_q8: null context");
  if (!c->kv_bits) return fail(CBD_E_UNSUPPORTED, "kvslab_read_q8: the context stores bf16 slabs");
  const Slab* s;
  if (cbd_status st = live_slab(c, seq_id, &s)) return st;
  if (start < 0 || n_tokens < 0) return fail(CBD_E_INVAL, "kvslab_read_q8: negative range");
  if ((int64_t)start + n_tokens > s->len)
    return fail(CBD_E_CAPACITY, "kvslab_read_q8: [%d, %d) beyond length %d", start, start + n_tokens, s->len);
  if (n_tokens == 0) return CBD_OK;
  if (!codes_out_dev || !sb_out_dev || !aligned16(codes_out_dev) || !aligned16(sb_out_dev))
    return fail(CBD_E_INVAL, "kvslab_read_q8: outputs must be 16-byte aligned device pointers");
  if (c->host_only) return fail(CBD_E_NODEVICE, "kvslab_read_q8: host-only context");
  const RowMeta m = row_meta(c, *s, start);
  const int32_t end = start + n_tokens, cut = std::min(std::max(start, m.pre_end), end);
  if (cut > start)
    HIP_TRY(launch_slab_q8(c->arena, m.pre_off, m.pre_stride, start, cut - start, n_tokens, 0, c->cfg.n_layers,
                           c->cfg.n_kv_heads, c->cfg.head_dim, nullptr, nullptr, static_cast<uint8_t*>(codes_out_dev),
                           static_cast<float*>(sb_out_dev), c->kv_bits, static_cast<hipStream_t>(stream)),
            "kvslab_read_q8 launch");
  if (end > cut)
    HIP_TRY(launch_slab_q8(c->arena, m.slab_off, s->stride, cut, end - cut, n_tokens, cut - start, c->cfg.n_layers,
                           c->cfg.n_kv_heads, c->cfg.head_dim, nullptr, nullptr, static_cast<uint8_t*>(codes_out_dev),
                           static_cast<float*>(sb_out_dev), c->kv_bits, static_cast<hipStream_t>(stream)),
            "kvslab_read_q8 launch");
  return CBD_OK;
}

// ----------------------------------------------------------------------------- the layer stack

namespace {

SkinnyArgs gemm_args(const cbd_ctx* c, const uint16_t* x, int64_t x_plane, int K, int rows,
                     std::initializer_list<Mat> segs, std::initializer_list<int> seg_rows, int N) {
  SkinnyArgs a{};
  a.x = x;
  a.x_plane = x_plane;
  a.K = K;
  a.rows = rows;
  a.N = N;
  int i = 0, acc = 0;
  auto r = seg_rows.begin();
  for (const Mat& m : segs) {
    a.w[i] = m.data;
    a.aux[i] = m.aux;
    acc += *r++;
    a.seg_end[i] = acc;
    ++i;
  }
  for (; i < 3; ++i) a.seg_end[i] = 0x7FFFFFFF;
  (void)c;
  return a;
}

// Plan and launch one weight-streaming product; the plan's workspace is checked against the context's.
hipError_t run_gemm(cbd_ctx* c, SkinnyArgs a, int epi, int x_blocks, int splits, hipStream_t st) {
  const SkinnyPlan p = plan_skinny(epi, c->fmt, a.N, a.K, a.rows, x_blocks, splits);
  if (skinny_part_bytes(p) > c->gemm_part_bytes || (p.splits > 1 && p.row_blocks > c->gemm_counter_count))
    return hipErrorInvalidValue;
  a.part = c->gemm_part;
  a.counters = c->gemm_counters;
  return launch_skinny_gemm(a, epi, c->fmt, x_blocks, p, st);
}

// The consumer of a norm: accumulators scaled by 1/rms of each activation row.
void with_norm(const cbd_ctx* c, SkinnyArgs& a) {
  a.ss = c->ss;
  a.ss_tiles = c->cfg.d_model / 16;
  a.ss_ld = c->rows_pad;
  a.norm_dim = (float)c->cfg.d_model;
  a.eps = c->cfg.rms_eps;
}

// A residual producer: h += y, then planes of next_gain * h and sums of squares for the next norm.
void with_residual(cbd_ctx* c, SkinnyArgs& a, const uint16_t* next_gain) {
  a.out = c->h;
  a.ldo = c->cfg.d_model;
  a.out_x = c->xa;
  a.out_plane = c->xa_plane;
  a.next_gain = next_gain;
  a.ss_out = c->ss;
  a.ss_out_ld = c->rows_pad;
}

// Algorithmic bytes of one weight-streaming launch: weights, the activation pair read (hi + lo bf16
// = 4 bytes per element), and what the epilogue writes: fp32 outputs (store), the residual read and
// written plus the next activation pair (residual), or the SwiGLU activation pair (swiglu).
double gemm_bytes(const cbd_ctx* c, int rows, int n_total, int K, int epi) {
  const double w = c->fmt == FMT_INT4 ? (double)n_total * K / 2 + (double)n_total * (K / 64) * 4
                                      : (double)n_total * K * 2;
  const double out = epi == EPI_SWIGLU ? (double)rows * (n_total / 2) * 4
                                       : (double)rows * n_total * (epi == EPI_RESIDUAL ? 12 : 4);
  return w + (double)rows * K * 4 + out;
}

double gemm_flops(int rows, int n_total, int K) { return 2.0 * rows * n_total * K; }

// Every layer for `rows` query rows whose metadata/items are already on the device.
// kv_keys: total keys attended per KV head over all items (for byte accounting).
cbd_status run_layers(cbd_ctx* c, int rows, int x_blocks, const RowMeta* meta_d, const AttnItem* items_d, int n_items,
                      const int32_t* row_parts_d, int n_parts, double kv_keys, hipStream_t st) {
  const cbd_model_config& m = c->cfg;
  for (int l = 0; l < m.n_layers; ++l) {
    const LayerW& L = c->layers[l];
    SkinnyArgs a = gemm_args(c, c->xa, c->xa_plane, m.d_model, rows, {L.wq, L.wk, L.wv},
                             {c->q_dim, c->kv_dim, c->kv_dim}, c->qkv_dim);
    with_norm(c, a);
    a.out = c->qkv;
    a.ldo = c->qkv_dim;
    {
      ProfScope p(c, CBD_KERNEL_QKV, gemm_bytes(c, rows, c->qkv_dim, m.d_model, EPI_STORE),
                  gemm_flops(rows, c->qkv_dim, m.d_model), st);
      HIP_TRY(run_gemm(c, a, EPI_STORE, x_blocks, 0, st), "qkv projection");
    }
    // decode rotates q and appends K/V inside the attention kernel; the prefill appends every
    // token's K/V first (its queries read each other's keys)
    const bool fused = row_parts_d != nullptr;
    if (!fused) {
      ProfScope p(c, CBD_KERNEL_ROPE_APPEND, (double)rows * (c->qkv_dim * 4.0 + c->q_dim * 4.0 + c->kv_dim * 4.0), 0, st);
      HIP_TRY(c->kv_bits ? launch_rope_append_q8(c->qkv, c->qkv_dim, meta_d, rows, m.n_heads, m.n_kv_heads,
                                                 m.head_dim, l, c->arena, c->rope_cs, c->kv_bits, st)
                         : launch_rope_append(c->qkv, c->qkv_dim, meta_d, rows, m.n_heads, m.n_kv_heads, m.head_dim,
                                              l, c->arena, c->rope_cs, st),
              "rope/append");
    }
    {
      AttnArgs at{};
      at.qkv = c->qkv;
      at.ld_qkv = c->qkv_dim;
      at.meta = meta_d;
      at.items = items_d;
      at.n_heads = m.n_heads;
      at.n_kv_heads = m.n_kv_heads;
      at.layer = l;
      at.arena = c->arena;
      at.rope_cs = reinterpret_cast<const float2*>(c->rope_cs);
      at.out = c->xo;
      at.out_plane = c->xo_plane;
      at.ld_out = c->q_dim;
      at.part_o = c->part_o;
      at.part_ml = c->part_ml;
      at.row_parts = reinterpret_cast<const int2*>(row_parts_d);
      at.counters = c->attn_counters;
      const double kvb = kv_keys * (c->kv_bits ? m.n_kv_heads * (m.head_dim * c->kv_bits / 8.0 + m.head_dim / kQGroup * 8.0) * 2.0
                                           : c->kv_dim * 2.0 * 2.0);
      ProfScope p(c, CBD_KERNEL_ATTENTION, kvb + (double)rows * c->q_dim * (4.0 + 4.0) + n_parts * 0.0,
                  kv_keys * m.n_heads * m.head_dim * 4.0, st);
      HIP_TRY(fused ? (c->kv_bits ? launch_decode_attention_q8(at, n_items, m.head_dim, c->kv_bits, st)
                              : launch_decode_attention(at, n_items, m.head_dim, st))
                    : (c->kv_bits ? launch_prefill_attention_q8(at, n_items, m.head_dim, c->kv_bits, st)
                              : launch_prefill_attention(at, n_items, m.head_dim, st)),
              "attention");
    }
    a = gemm_args(c, c->xo, c->xo_plane, c->q_dim, rows, {L.wo}, {m.d_model}, m.d_model);
    with_residual(c, a, L.ffn_norm);
    {
      ProfScope p(c, CBD_KERNEL_O_PROJ, gemm_bytes(c, rows, m.d_model, c->q_dim, EPI_RESIDUAL),
                  gemm_flops(rows, m.d_model, c->q_dim), st);
      HIP_TRY(run_gemm(c, a, EPI_RESIDUAL, x_blocks, 0, st), "o projection");
    }
    a = gemm_args(c, c->xa, c->xa_plane, m.d_model, rows, {L.wg, L.wu}, {m.ffn_dim, m.ffn_dim}, m.ffn_dim);
    with_norm(c, a);
    a.out_x = c->xm;
    a.out_plane = c->xm_plane;
    a.ldo = m.ffn_dim;
    {
      ProfScope p(c, CBD_KERNEL_GATE_UP, gemm_bytes(c, rows, 2 * m.ffn_dim, m.d_model, EPI_SWIGLU),
                  gemm_flops(rows, 2 * m.ffn_dim, m.d_model), st);
      HIP_TRY(run_gemm(c, a, EPI_SWIGLU, x_blocks, 0, st), "gate/up projection");
    }
    a = gemm_args(c, c->xm, c->xm_plane, m.ffn_dim, rows, {L.wd}, {m.d_model}, m.d_model);
    with_residual(c, a, (l + 1 < m.n_layers) ? c->layers[l + 1].attn_norm : c->final_norm);
    {
      ProfScope p(c, CBD_KERNEL_DOWN, gemm_bytes(c, rows, m.d_model, m.ffn_dim, EPI_RESIDUAL),
                  gemm_flops(rows, m.d_model, m.ffn_dim), st);
      HIP_TRY(run_gemm(c, a, EPI_RESIDUAL, x_blocks, 0, st), "down projection");
    }
  }
  return CBD_OK;
}

// Final norm (folded into the product) + lm_head for `rows` rows; row_idx_d gathers the
// activation rows (prefill: each segment's last token) into compact rows first.
cbd_status run_head(cbd_ctx* c, const int32_t* row_idx_d, int rows, float* logits, int32_t* next_tokens,
                    hipStream_t st) {
  const cbd_model_config& m = c->cfg;
  const uint16_t* x = c->xa;
  int64_t x_plane = c->xa_plane;
  if (row_idx_d) {
    // the last layer's SwiGLU planes are consumed: reuse them for the gathered rows
    HIP_TRY(launch_gather_rows(c->xa, c->xa_plane, c->ss, c->rows_pad, row_idx_d, rows, m.d_model, c->xm, c->xm_plane,
                               c->ss_head, 64, st),
            "head row gather");
    x = c->xm;
    x_plane = c->xm_plane;
  }
  SkinnyArgs a = gemm_args(c, x, x_plane, m.d_model, rows, {c->lm_head}, {m.vocab}, m.vocab);
  with_norm(c, a);
  if (row_idx_d) {
    a.ss = c->ss_head;
    a.ss_ld = 64;
  }
  a.out = logits;
  a.ldo = m.vocab;
  {
    ProfScope p(c, CBD_KERNEL_LM_HEAD, gemm_bytes(c, rows, m.vocab, m.d_model, EPI_STORE),
                gemm_flops(rows, m.vocab, m.d_model), st);
    HIP_TRY(run_gemm(c, a, EPI_STORE, 1, 0, st), "lm_head");
  }
  if (next_tokens) {
    ProfScope p(c, CBD_KERNEL_ARGMAX, rows * (double)m.vocab * 4.0, 0, st);
    HIP_TRY(launch_argmax(logits, rows, m.vocab, c->argmax_part, c->argmax_counters, next_tokens, st), "argmax");
  }
  return CBD_OK;
}

}  // namespace

// ----------------------------------------------------------------------------- hot path

extern "C" cbd_status decode_step_batch(cbd_ctx* c, const int32_t* seq_ids, int32_t B, const int32_t* last_tokens_dev,
                                        float* logits_dev, int32_t* next_tokens_dev, cbd_stream stream) {
  if (!c) return fail(CBD_E_INVAL, "decode_step_batch: null context");
  if (B < 0 || B > c->lim.max_batch) return fail(CBD_E_INVAL, "decode_step_batch: B=%d outside 0..%d", B, c->lim.max_batch);
  if (B == 0) return CBD_OK;
  if (!seq_ids || !last_tokens_dev || !logits_dev) return fail(CBD_E_INVAL, "decode_step_batch: null pointer");
  if (!aligned16(logits_dev)) return fail(CBD_E_INVAL, "decode_step_batch: logits must be 16-byte aligned");
  std::vector<RowMeta> rows(B);
  for (int i = 0; i < B; ++i) {
    const Slab* s;
    if (cbd_status st = live_slab(c, seq_ids[i], &s)) return st;
    for (int j = 0; j < i; ++j)
      if (seq_ids[j] == seq_ids[i]) return fail(CBD_E_INVAL, "decode_step_batch: duplicate sequence id %d", seq_ids[i]);
    if (s->len + 1 > s->cap)
      return fail(CBD_E_CAPACITY, "decode_step_batch: sequence %d is full (%d tokens)", seq_ids[i], s->cap);
    if (s->len + 1 > c->cfg.max_position)
      return fail(CBD_E_CAPACITY, "decode_step_batch: sequence %d reached max_position", seq_ids[i]);
    rows[i] = row_meta(c, *s, s->len);
  }
  if (c->host_only) return fail(CBD_E_NODEVICE, "decode_step_batch: host-only context");
  hipStream_t st = static_cast<hipStream_t>(stream);
  int slot;
  uint8_t* host = staging_slot(c, &slot);
  // packed per-call layout: rows | items | row_parts (offsets rounded to 256 bytes)
  const size_t items_off = round_up((int64_t)B * sizeof(RowMeta), 256);
  AttnItem* items = reinterpret_cast<AttnItem*>(host + items_off);
  std::vector<int32_t> row_parts(2 * B);
  std::memcpy(host, rows.data(), B * sizeof(RowMeta));
  const int n_items = plan_decode_items(c, rows, items, row_parts.data());
  const size_t parts_off = round_up(items_off + (size_t)n_items * sizeof(AttnItem), 256);
  std::memcpy(host + parts_off, row_parts.data(), row_parts.size() * sizeof(int32_t));
  int n_parts = 0;
  for (int i = 0; i < B; ++i) n_parts += row_parts[2 * i + 1];
  double kv_keys = 0;
  for (int i = 0; i < B; ++i) kv_keys += rows[i].pos + 1;
  if (cbd_status s = upload(c, slot, parts_off + row_parts.size() * sizeof(int32_t), st)) return s;
  const RowMeta* meta_d = reinterpret_cast<const RowMeta*>(c->meta_dev);
  const AttnItem* items_d = reinterpret_cast<const AttnItem*>(c->meta_dev + items_off);
  const int32_t* parts_d = reinterpret_cast<const int32_t*>(c->meta_dev + parts_off);

  const cbd_model_config& m = c->cfg;
  {
    ProfScope p(c, CBD_KERNEL_EMBED, B * (double)m.d_model * 12.0, 0, st);
    HIP_TRY(launch_embed(last_tokens_dev, B, c->embed, m.vocab, m.d_model, c->layers[0].attn_norm, c->h, c->xa,
                         c->xa_plane, c->ss, c->rows_pad, st),
            "embed");
  }
  if (cbd_status s = run_layers(c, B, 1, meta_d, items_d, n_items, parts_d, n_parts, kv_keys, st)) return s;
  if (cbd_status s = run_head(c, nullptr, B, logits_dev, next_tokens_dev, st)) return s;
  for (int i = 0; i < B; ++i) c->slabs[seq_ids[i]].len += 1;
  c->stats.decode_steps += 1;
  c->stats.decode_rows += B;
  return CBD_OK;
}

extern "C" cbd_status prefill_segmented(cbd_ctx* c, const int32_t* seq_ids, const int32_t* seg_lens, int32_t K,
                                        const int32_t* tokens_dev, float* last_logits_dev, int32_t* next_tokens_dev,
                                        cbd_stream stream) {
  if (!c) return fail(CBD_E_INVAL, "prefill_segmented: null context");
  if (K < 0 || K > c->lim.max_segments)
    return fail(CBD_E_INVAL, "prefill_segmented: K=%d outside 0..%d", K, c->lim.max_segments);
  if (K == 0) return CBD_OK;
  if (!seq_ids || !seg_lens || !tokens_dev || !last_logits_dev) return fail(CBD_E_INVAL, "prefill_segmented: null pointer");
  if (!aligned16(last_logits_dev)) return fail(CBD_E_INVAL, "prefill_segmented: logits must be 16-byte aligned");
  int64_t T = 0;
  for (int i = 0; i < K; ++i) {
    const Slab* s;
    if (cbd_status st = live_slab(c, seq_ids[i], &s)) return st;
    for (int j = 0; j < i; ++j)
      if (seq_ids[j] == seq_ids[i]) return fail(CBD_E_INVAL, "prefill_segmented: duplicate sequence id %d", seq_ids[i]);
    if (seg_lens[i] < 1) return fail(CBD_E_INVAL, "prefill_segmented: segment %d has length %d", i, seg_lens[i]);
    // a segment continues its sequence: positions len .. len + L - 1 (len = 0 for a fresh slab)
    if ((int64_t)s->len + seg_lens[i] > s->cap || (int64_t)s->len + seg_lens[i] > c->cfg.max_position)
      return fail(CBD_E_CAPACITY, "prefill_segmented: %d tokens after %d exceed slab %d (capacity %d)", seg_lens[i],
                  s->len, seq_ids[i], s->cap);
    T += seg_lens[i];
  }
  if (T > c->lim.max_prefill_tokens)
    return fail(CBD_E_INVAL, "prefill_segmented: %lld tokens exceed max_prefill_tokens %d", (long long)T,
                c->lim.max_prefill_tokens);
  if (c->host_only) return fail(CBD_E_NODEVICE, "prefill_segmented: host-only context");
  hipStream_t st = static_cast<hipStream_t>(stream);
  int slot;
  uint8_t* host = staging_slot(c, &slot);
  // packed per-call layout: rows | items | last-token row indices
  const size_t items_off = round_up(T * (int64_t)sizeof(RowMeta), 256);
  const size_t idx_off = round_up(items_off + T * sizeof(AttnItem), 256);
  RowMeta* rows = reinterpret_cast<RowMeta*>(host);
  AttnItem* items = reinterpret_cast<AttnItem*>(host + items_off);
  int32_t* last_idx = reinterpret_cast<int32_t*>(host + idx_off);
  // attention items: tiles of up to 16 consecutive queries of one segment (keys 0 .. end of tile:
  // the sequence's earlier keys, then the segment's own up to each query), the longest first so the
  // grid's tail is short
  int g = 0, n_items = 0;
  for (int i = 0; i < K; ++i) {
    const Slab& s = c->slabs[seq_ids[i]];
    const int t0 = s.len;
    for (int p = 0; p < seg_lens[i]; ++p) rows[g + p] = row_meta(c, s, t0 + p);
    const RowMeta& m = rows[g];
    for (int p0 = 0; p0 < seg_lens[i]; p0 += 16)
      items[n_items++] = AttnItem{m.slab_off, m.stride, t0 + p0, g + p0, 0, t0 + std::min(p0 + 16, seg_lens[i]), -1,
                                  m.pre_off, m.pre_stride, m.pre_end};
    g += seg_lens[i];
    last_idx[i] = g - 1;
  }
  std::stable_sort(items, items + n_items, [](const AttnItem& x, const AttnItem& y) { return x.k_end > y.k_end; });
  if (cbd_status s = upload(c, slot, idx_off + K * sizeof(int32_t), st)) return s;
  const RowMeta* meta_d = reinterpret_cast<const RowMeta*>(c->meta_dev);
  const AttnItem* items_d = reinterpret_cast<const AttnItem*>(c->meta_dev + items_off);
  const int32_t* idx_d = reinterpret_cast<const int32_t*>(c->meta_dev + idx_off);

  const cbd_model_config& m = c->cfg;
  const int x_blocks = (int)((T + 63) / 64);
  double kv_keys = 0;
  for (int i = 0; i < K; ++i)
    kv_keys += (double)seg_lens[i] * c->slabs[seq_ids[i]].len + 0.5 * (double)seg_lens[i] * (seg_lens[i] + 1);
  {
    ProfScope p(c, CBD_KERNEL_EMBED, T * (double)m.d_model * 12.0, 0, st);
    HIP_TRY(launch_embed(tokens_dev, (int)T, c->embed, m.vocab, m.d_model, c->layers[0].attn_norm, c->h, c->xa,
                         c->xa_plane, c->ss, c->rows_pad, st),
            "embed");
  }
  if (cbd_status s = run_layers(c, (int)T, x_blocks, meta_d, items_d, n_items, nullptr, 0, kv_keys, st)) return s;
  if (cbd_status s = run_head(c, idx_d, K, last_logits_dev, next_tokens_dev, st)) return s;
  for (int i = 0; i < K; ++i) c->slabs[seq_ids[i]].len += seg_lens[i];
  c->stats.prefill_calls += 1;
  c->stats.prefill_tokens += T;
  return CBD_OK;
}

extern "C" cbd_status greedy_argmax(cbd_ctx* c, const float* logits_dev, int32_t rows, int32_t* tokens_dev,
                                    cbd_stream stream) {
  if (!c) return fail(CBD_E_INVAL, "greedy_argmax: null context");
  if (rows < 0 || rows > 64) return fail(CBD_E_INVAL, "greedy_argmax: rows must be in 0..64");
  if (rows == 0) return CBD_OK;
  if (!logits_dev || !tokens_dev || !aligned16(logits_dev)) return fail(CBD_E_INVAL, "greedy_argmax: bad pointer");
  if (c->host_only) return fail(CBD_E_NODEVICE, "greedy_argmax: host-only context");
  HIP_TRY(launch_argmax(logits_dev, rows, c->cfg.vocab, c->argmax_part, c->argmax_counters, tokens_dev,
                        static_cast<hipStream_t>(stream)), "argmax");
  return CBD_OK;
}

extern "C" cbd_status sample_top_p(cbd_ctx* c, const float* logits_dev, int32_t rows, const float* temperature,
                                   const float* top_p, const uint64_t* seeds, const uint64_t* sample_index,
                                   int32_t* tokens_dev, cbd_stream stream) {
  if (!c) return fail(CBD_E_INVAL, "sample_top_p: null context");
  if (rows < 0 || rows > 64) return fail(CBD_E_INVAL, "sample_top_p: rows must be in 0..64");
  if (rows == 0) return CBD_OK;
  if (!logits_dev || !tokens_dev || !temperature || !top_p || !seeds || !sample_index || !aligned16(logits_dev))
    return fail(CBD_E_INVAL, "sample_top_p: null or unaligned pointer");
  if (c->cfg.vocab % 4) return fail(CBD_E_INVAL, "sample_top_p: vocab %d is not a multiple of 4", c->cfg.vocab);
  SampleArgs a{};
  for (int r = 0; r < rows; ++r) {
    if (!(temperature[r] >= 0.f) || !std::isfinite(temperature[r]))
      return fail(CBD_E_INVAL, "sample_top_p: row %d temperature %g", r, (double)temperature[r]);
    if (!(top_p[r] > 0.f && top_p[r] <= 1.f)) return fail(CBD_E_INVAL, "sample_top_p: row %d top_p %g", r, (double)top_p[r]);
    a.temperature[r] = temperature[r];
    a.top_p[r] = top_p[r];
    a.seed[r] = seeds[r];
    a.index[r] = sample_index[r];
  }
  if (c->host_only) return fail(CBD_E_NODEVICE, "sample_top_p: host-only context");
  hipStream_t st = static_cast<hipStream_t>(stream);
  ProfScope p(c, CBD_KERNEL_SAMPLE, (double)rows * c->cfg.vocab * 4.0, 0, st);
  HIP_TRY(launch_sample_top_p(logits_dev, rows, c->cfg.vocab, a, c->sample_ws, tokens_dev, st), "sample_top_p");
  return CBD_OK;
}

extern "C" cbd_status cbd_linear(cbd_ctx* c, const cbd_matrix* w, int32_t N, int32_t K, const float* x_dev,
                                 int32_t rows, float* y_dev, int32_t splits, cbd_stream stream) {
  if (!c || !w || !x_dev || !y_dev) return fail(CBD_E_INVAL, "cbd_linear: null argument");
  if (rows < 1 || rows > 64) return fail(CBD_E_INVAL, "cbd_linear: rows must be in 1..64");
  if (N < 64 || N % 64) return fail(CBD_E_INVAL, "cbd_linear: N must be a positive multiple of 64");
  if (K < 1 || !skinny_shape_ok(c->fmt, K))
    return fail(CBD_E_INVAL, "cbd_linear: K=%d not supported for this weight format", K);
  if (K > std::max(c->cfg.ffn_dim, c->cfg.d_model)) return fail(CBD_E_INVAL, "cbd_linear: K above the model width");
  if (splits > 64 || (splits > 0 && (K % splits || (K / splits) % 128)))
    return fail(CBD_E_INVAL, "cbd_linear: splits must divide K into multiples of 128 inputs");
  if (splits < 0 && splits != -4 && splits != -8 && splits != -16)
    return fail(CBD_E_INVAL, "cbd_linear: a k split takes 4, 8 or 16 waves");
  if (splits < 0) {  // the k-split kernel's limits: row groups per wave, and two stages per wave
    const bool int4 = c->fmt == FMT_INT4;
    const int step = int4 ? 128 : 32;
    if ((int4 && rows > 16) || (splits == -16 && rows > 8) || (int4 && splits < -4 && rows > 8) ||
        K / (-splits) < 2 * step || K % (-splits * step))
      return fail(CBD_E_INVAL, "cbd_linear: a %d-wave k split does not fit rows=%d, K=%d", -splits, rows, K);
  }
  if (!w->data || !aligned16(w->data) || (c->fmt == FMT_INT4 && (!w->aux || !aligned16(w->aux))) ||
      !aligned16(y_dev) || !aligned16(x_dev))
    return fail(CBD_E_INVAL, "cbd_linear: pointers must be 16-byte aligned");
  if (c->host_only) return fail(CBD_E_NODEVICE, "cbd_linear: host-only context");
  hipStream_t st = static_cast<hipStream_t>(stream);
  // split the rows into hi/lo planes in the padded workspace (the column tile never reads past it)
  HIP_TRY(launch_split_planes(static_cast<const float*>(x_dev), rows, K, c->xm, c->xm_plane, st), "cbd_linear split");
  SkinnyArgs a = gemm_args(c, c->xm, c->xm_plane, K, rows, {Mat{w->data, w->aux}}, {N}, N);
  a.out = y_dev;
  a.ldo = N;
  HIP_TRY(run_gemm(c, a, EPI_STORE, 1, splits, st), "cbd_linear");
  return CBD_OK;
}

extern "C" cbd_status cbd_pack_int4(const uint8_t* codes, const uint16_t* scale, const uint16_t* bias, int64_t N,
                                    int64_t K, uint32_t* packed_out, uint16_t* aux_out) {
  if (!codes || !scale || !bias || !packed_out || !aux_out) return fail(CBD_E_INVAL, "cbd_pack_int4: null argument");
  if (N < 1 || K < 128 || K % 128 || N % 16) return fail(CBD_E_INVAL, "cbd_pack_int4: need K % 128 == 0 and N % 16 == 0");
  const int64_t G = K / 64, blocks = K / 128;
  for (int64_t n = 0; n < N; ++n) {
    const uint8_t* row = codes + n * K;
    const int64_t tr = n / 16, r = n % 16;
    for (int64_t b = 0; b < blocks; ++b)
      for (int g = 0; g < 4; ++g) {
        uint32_t* lane_words = packed_out + ((tr * blocks + b) * 64 + (16 * g + r)) * 4;
        for (int j = 0; j < 4; ++j) {
          uint32_t word = 0;
          const int64_t base = b * 128 + 32 * j + 8 * g;
          for (int e = 0; e < 8; ++e) {
            const uint32_t q = row[base + e];
            if (q > 15) return fail(CBD_E_INVAL, "cbd_pack_int4: code %u out of range", q);
            word |= q << (4 * ((e >> 1) + 4 * (e & 1)));
          }
          lane_words[j] = word;
        }
      }
    for (int64_t gi = 0; gi < G; ++gi) {
      aux_out[(gi * N + n) * 2 + 0] = scale[n * G + gi];
      aux_out[(gi * N + n) * 2 + 1] = bias[n * G + gi];
    }
  }
  return CBD_OK;
}

extern "C" cbd_status cbd_pack_bf16(const void* src_dev, int64_t N, int64_t K, void* dst_dev, cbd_stream stream) {
  if (!src_dev || !dst_dev || !aligned16(src_dev) || !aligned16(dst_dev))
    return fail(CBD_E_INVAL, "cbd_pack_bf16: pointers must be 16-byte aligned device pointers");
  if (N < 16 || N % 16 || K < 32 || K % 32) return fail(CBD_E_INVAL, "cbd_pack_bf16: need N % 16 == 0 and K % 32 == 0");
  if (src_dev == dst_dev) return fail(CBD_E_INVAL, "cbd_pack_bf16: source and destination must differ");
  HIP_TRY(launch_pack_bf16(static_cast<const uint16_t*>(src_dev), N, K, static_cast<uint16_t*>(dst_dev),
                           static_cast<hipStream_t>(stream)),
          "cbd_pack_bf16 launch");
  return CBD_OK;
}

extern "C" cbd_status cbd_profile_begin(cbd_ctx* c, uint32_t kind_mask, int32_t max_launches, int32_t every) {
  if (!c) return fail(CBD_E_INVAL, "cbd_profile_begin: null context");
  if (max_launches < 0 || max_launches > (1 << 22)) return fail(CBD_E_INVAL, "cbd_profile_begin: bad max_launches");
  if (every < 1) return fail(CBD_E_INVAL, "cbd_profile_begin: every must be >= 1");
  if (c->host_only) return fail(CBD_E_NODEVICE, "cbd_profile_begin: host-only context");
  while ((int)c->prof_ev.size() < 2 * max_launches) {
    hipEvent_t e;
    HIP_TRY(hipEventCreate(&e), "profile event create");
    c->prof_ev.push_back(e);
  }
  c->prof_rec.clear();
  c->prof_max = max_launches;
  c->prof_every = every;
  c->prof_seen = 0;
  c->prof_mask = kind_mask;
  return CBD_OK;
}

extern "C" cbd_status cbd_profile_end(cbd_ctx* c, cbd_kernel_time* out) {
  if (!c || !out) return fail(CBD_E_INVAL, "cbd_profile_end: null argument");
  for (int k = 0; k < CBD_KERNEL_KINDS; ++k) out[k] = cbd_kernel_time{0, 0.0, 0.0, 0.0};
  c->prof_mask = 0;
  if (c->prof_rec.empty()) return CBD_OK;
  HIP_TRY(hipEventSynchronize(c->prof_ev[2 * c->prof_rec.size() - 1]), "profile wait");
  for (size_t i = 0; i < c->prof_rec.size(); ++i) {
    float ms = 0.f;
    HIP_TRY(hipEventElapsedTime(&ms, c->prof_ev[2 * i], c->prof_ev[2 * i + 1]), "profile elapsed");
    cbd_kernel_time& t = out[c->prof_rec[i].kind];
    t.launches += 1;
    t.total_ms += ms;
    t.bytes += c->prof_rec[i].bytes;
    t.flops += c->prof_rec[i].flops;
  }
  c->prof_rec.clear();
  return CBD_OK;
}

// Host planner: validation of the configuration and batch, and the split of the hybrid batch
// into work items.
//
// Prefill: each chunk is cut into query tiles of floor(128 / group) rows, so that one tile is
// 128 (query, head) columns sharing one KV head; a tile needs the keys up to its last query's
// position.  Long tiles are split along the keys into at most `prefill_split_cap` ranges, the
// cap that keeps one prefill chunk from flooding the machine with work items and pushing
// decode out (Silicon & Systems, "POD-Attention hybrid batching", section "Virtual CTAs and
// per-SM balance").
// Decode: each (sequence, KV head) is split along its context into ranges of about
// `decode_split_tokens` keys whose partial results are merged by log-sum-exp ("LLMSO - W4 -
// Optimization & Frameworks", section "FlashDecoding -- decode 단계의 병렬성 확보"); the split
// length is chosen from the total decode work and the number of persistent workgroups so that
// every workgroup gets many small items and the last wave of work stays short (the wave
// quantization loss of the same digest, section "Why concurrency alone is not enough").
// Decode work is ordered longest first; prefill work is dealt to per-XCD queues (below).
#include "plan.h"

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstring>
#include <numeric>

namespace pod {

namespace {
// Sustained rates of the two shares on gfx950, used only to tell a prefill-heavy batch from a
// decode-heavy one when sizing decode splits: the prefill tile at about a third of the bf16
// matrix peak, the decode stream at about 6.5 TB/s (both measured with rocprofv3).
constexpr double kPrefillFlopsPerSec = 0.85e15;
constexpr double kDecodeBytesPerSec = 6.5e12;
constexpr double kPrefillHeavyRatio = 0.75;   // prefill share >= 3/4 of the decode share
constexpr int kOneRoundMaxSplit = 8192;       // longest decode split of the prefill-heavy fused plan
constexpr int kOneRoundMaxSplitFp8 = 5120;    // the same with an FP8 cache
constexpr int kMinDecodeSplit = 256;          // shortest decode split the planner chooses
constexpr int kMinPrefillSplit = 4096;        // shortest key split of a prefill tile
int ceil_div(long a, long b) { return (int)((a + b - 1) / b); }
int round_up_int(int a, int m) { return ceil_div(a, m) * m; }
}  // namespace

pod_attn_status validate_config(const pod_attn_config* c, Config* out, std::string* err) {
  if (!c || !out) { *err = "null config"; return POD_ATTN_ERR_INVALID_ARG; }
  if (c->num_q_heads < 1 || c->num_kv_heads < 1) {
    *err = "num_q_heads and num_kv_heads must be >= 1"; return POD_ATTN_ERR_INVALID_ARG;
  }
  if (c->num_q_heads % c->num_kv_heads != 0) {
    *err = "num_q_heads must be a multiple of num_kv_heads"; return POD_ATTN_ERR_INVALID_ARG;
  }
  if (c->num_q_heads / c->num_kv_heads > kMaxGroup) {
    *err = "query heads per KV head above 16 are not supported"; return POD_ATTN_ERR_UNSUPPORTED;
  }
  if (c->page_size != kPage) { *err = "page_size must be 16"; return POD_ATTN_ERR_UNSUPPORTED; }
  if (c->head_dim != 64 && c->head_dim != 128) {
    *err = "head_dim must be 64 or 128"; return POD_ATTN_ERR_UNSUPPORTED;
  }
  if (c->dtype != POD_ATTN_BF16 && c->dtype != POD_ATTN_FP32 && c->dtype != POD_ATTN_FP8_E4M3) {
    *err = "dtype must be POD_ATTN_BF16, POD_ATTN_FP32 or POD_ATTN_FP8_E4M3"; return POD_ATTN_ERR_INVALID_ARG;
  }
  if (c->mode < POD_ATTN_MODE_FUSED || c->mode > POD_ATTN_MODE_STREAMS) {
    *err = "unknown mode"; return POD_ATTN_ERR_INVALID_ARG;
  }
  if (!(c->scale >= 0.f) || std::isinf(c->scale)) {
    *err = "scale must be finite and >= 0"; return POD_ATTN_ERR_INVALID_ARG;
  }
  if (c->decode_split_tokens < 0 || (c->decode_split_tokens % 128) != 0) {
    *err = "decode_split_tokens must be 0 or a positive multiple of 128"; return POD_ATTN_ERR_INVALID_ARG;
  }
  if (c->prefill_split_cap < 0 || c->prefill_split_cap > kMaxCombineSplits || c->wgs_per_cu < 0 || c->wgs_per_cu > 8) {
    *err = "prefill_split_cap must be in [0, 128] and wgs_per_cu in [0, 8]"; return POD_ATTN_ERR_INVALID_ARG;
  }
  if (c->extend_max_q < -1 || c->extend_max_q > 256) {
    *err = "extend_max_q must be -1, 0 or in [1, 256]"; return POD_ATTN_ERR_INVALID_ARG;
  }
  Config k;
  k.hq = c->num_q_heads; k.hkv = c->num_kv_heads; k.d = c->head_dim; k.page = c->page_size;
  k.dtype = c->dtype; k.mode = c->mode;
  k.scale = c->scale > 0.f ? c->scale : 1.0f / std::sqrt((float)c->head_dim);
  k.decode_split_tokens = c->decode_split_tokens; k.prefill_split_cap = c->prefill_split_cap;
  k.wgs_per_cu = c->wgs_per_cu; k.flags = c->flags; k.extend_max_q = c->extend_max_q;
  *out = k;
  return POD_ATTN_OK;
}

pod_attn_status plan_batch(const Config& c, const pod_attn_batch* b, int num_cus, int wgs_per_cu,
                           Plan* out, std::string* err) {
  if (!b) { *err = "null batch"; return POD_ATTN_ERR_INVALID_ARG; }
  if (b->num_prefill < 0 || b->num_decode < 0) { *err = "negative sequence count"; return POD_ATTN_ERR_INVALID_ARG; }
  if (b->num_prefill > 0 && (!b->prefill_q_start || !b->prefill_ctx_len)) {
    *err = "prefill arrays are null"; return POD_ATTN_ERR_INVALID_ARG;
  }
  if (b->num_decode > 0 && !b->decode_ctx_len) { *err = "decode_ctx_len is null"; return POD_ATTN_ERR_INVALID_ARG; }
  if (b->block_table_stride < 1) { *err = "block_table_stride must be >= 1"; return POD_ATTN_ERR_INVALID_ARG; }
  if (b->num_pages_in_pool < 1) { *err = "num_pages_in_pool must be >= 1"; return POD_ATTN_ERR_INVALID_ARG; }
  if (num_cus < 1 || wgs_per_cu < 1) { *err = "bad device shape"; return POD_ATTN_ERR_INVALID_ARG; }
  const long max_ctx = (long)b->block_table_stride * kPage;
  if (b->num_prefill > 0 && b->prefill_q_start[0] != 0) {
    *err = "prefill_q_start[0] must be 0"; return POD_ATTN_ERR_INVALID_ARG;
  }
  for (int i = 0; i < b->num_prefill; ++i) {
    long L = (long)b->prefill_q_start[i + 1] - b->prefill_q_start[i];
    long ctx = b->prefill_ctx_len[i];
    if (L < 0) { *err = "prefill_q_start must be non-decreasing (chunk " + std::to_string(i) + ")"; return POD_ATTN_ERR_INVALID_ARG; }
    if (ctx < L) { *err = "prefill chunk " + std::to_string(i) + ": q_len exceeds ctx"; return POD_ATTN_ERR_INVALID_ARG; }
    if (ctx > max_ctx) { *err = "prefill chunk " + std::to_string(i) + ": ctx exceeds block_table_stride*16"; return POD_ATTN_ERR_INVALID_ARG; }
    if (ctx > (1L << 30)) { *err = "context too long"; return POD_ATTN_ERR_INVALID_ARG; }
  }
  for (int i = 0; i < b->num_decode; ++i) {
    long ctx = b->decode_ctx_len[i];
    if (ctx < 1) { *err = "decode " + std::to_string(i) + ": ctx must be >= 1"; return POD_ATTN_ERR_INVALID_ARG; }
    if (ctx > max_ctx) { *err = "decode " + std::to_string(i) + ": ctx exceeds block_table_stride*16"; return POD_ATTN_ERR_INVALID_ARG; }
    if (ctx > (1L << 30)) { *err = "context too long"; return POD_ATTN_ERR_INVALID_ARG; }
  }
  const long prefill_rows = b->num_prefill > 0 ? (long)b->prefill_q_start[b->num_prefill] : 0;
  if (prefill_rows + b->num_decode > (1L << 30)) { *err = "too many query rows"; return POD_ATTN_ERR_INVALID_ARG; }

  Plan p;
  const int G = c.group();
  p.tile_queries = kTileCols / G;
  p.tile_cols = p.tile_queries * G;
  p.prefill_rows = (int)prefill_rows;
  p.total_q = (int)prefill_rows + b->num_decode;

  // ---------------- KV append units
  // Every query row's new token goes to its position's page slot before attention reads it
  // (a prefill chunk's L rows at ctx-L .. ctx-1, a decode row at ctx-1).  A sequence's new
  // tokens are cut at page boundaries into runs of consecutive slots, and each run into units
  // of about append_token_heads (token, KV head) pairs.
  auto add_units = [&](int seq, int row0, int pos0, int n) {
    for (int a = 0; a < n;) {
      const int pos = pos0 + a;
      const int ntok = std::min(n - a, kPage - pos % kPage);
      const int hg = std::max(1, std::min(c.hkv, c.append_token_heads / ntok));
      for (int h0 = 0; h0 < c.hkv; h0 += hg) {
        const int32_t u[kAUnitInts] = {seq, row0 + a, pos, ntok, h0, std::min(hg, c.hkv - h0), 0, 0};
        p.aunits.insert(p.aunits.end(), u, u + kAUnitInts);
      }
      a += ntok;
    }
  };
  for (int i = 0; i < b->num_decode; ++i)
    add_units(b->num_prefill + i, (int)prefill_rows + i, b->decode_ctx_len[i] - 1, 1);
  for (int i = 0; i < b->num_prefill; ++i) {
    const int L = b->prefill_q_start[i + 1] - b->prefill_q_start[i];
    if (L > 0) add_units(i, b->prefill_q_start[i], b->prefill_ctx_len[i] - L, L);
  }
  p.n_aunits = (int)(p.aunits.size() / kAUnitInts);

  // ---------------- prefill tiles
  // Tiles of one chunk share their split boundaries (one split length per chunk), so that the
  // tiles reading the same key range of the same KV head form a group.  Groups are dealt whole
  // to the kXcds per-XCD claim queues, largest first onto the least-loaded queue, so that a
  // group's tiles run together under one L2 and every XCD gets about the same work.
  struct Tile { int seq, q_row, n_q, q_pos, kv_len; };
  const int cap = c.prefill_split_cap > 0 ? c.prefill_split_cap : 8;
  int group = 0, slot = 0;
  p.prefill_max_splits = 0;
  struct PGroup { double work; std::vector<int32_t> items; };   // items: (desc, split << 16 | head)
  std::vector<PGroup> pgroups;
  // Small-q extends: a chunk whose rows x G fit one 16-column block (and of at most extend_max_q
  // rows) reads its whole prefix for a few queries, a decode-shaped, bandwidth-bound job; it runs
  // on the decode path ([W6] "한 스텝에 여러 종류의 request 섞기": a decode is an extend of one
  // token).  Longer chunks stay prefill tiles, which read the prefix once for 128 columns
  // (measured on 4-token to 16-token verification steps at G = 4: one block 1.3x faster than
  // a tile, two or more blocks that each re-read the prefix 1.3-2.2x slower).
  const int emax = c.extend_max_q < 0 ? 0 : (c.extend_max_q == 0 ? kExtendMaxQ : c.extend_max_q);
  const double kv_tok_bytes = 2.0 * c.hkv * c.d * c.elem_bytes();   // K and V of one token
  const double qo_row_bytes = 2.0 * c.hq * c.d * c.q_elem_bytes();  // q in and out of one row
  const double page_bytes = 4.0 + (c.dtype == POD_ATTN_FP8_E4M3 ? 8.0 * c.hkv : 0.0);   // table entry (+ FP8 scales)
  std::vector<int> small_chunks;
  auto is_small = [&](int L) { return L <= emax && L * G <= kMaxGroup; };
  // Key splits of a chunk's tiles.  A split costs a partial write, its read-back in the merge and
  // a pipeline fill, so tiles are split only as far as the workgroups that run them need: pieces
  // of at least kMinPrefillSplit keys, at most `cap` per tile.  When the tiles run beside a longer
  // decode stream (fused and two-stream modes, a batch that is not prefill-heavy by the estimate
  // below), about one workgroup per CU runs them, so a piece is also about the prefill share's
  // keys (all tiles, all KV heads) over the CUs: about one item per CU.  Measured (kernel us,
  // split caps 8 / 2 / 1): Llama-3-8B-shaped fused 1626 / 1563 / 1559, two-stream 1824 / 1731 /
  // 1696; long-context fused 5016 / 4987 / 5029, two-stream 5566 / 5130 / 5078.  A prefill-heavy
  // batch keeps the floor: its decode share ends early and every workgroup then runs tiles (the
  // Yi-6B-shaped batch, two-stream 587 / 607 / 888 us, and 573 -> 595 fused with an FP8 cache),
  // and so does separate mode, which runs tiles on every workgroup slot (Yi-6B-shaped: 695 us
  // against 818 at a cap of 2).
  double beside_split = 0.0;
  {
    double tile_keys = 0.0, pf_flops = 0.0, dc_bytes = 0.0;
    for (int i = 0; i < b->num_prefill; ++i) {
      const int L = b->prefill_q_start[i + 1] - b->prefill_q_start[i];
      const double ctx = b->prefill_ctx_len[i];
      if (L == 0) continue;
      if (is_small(L)) {
        dc_bytes += ctx * kv_tok_bytes + L * qo_row_bytes + page_bytes * ceil_div((int)ctx, kPage);
        continue;
      }
      for (int t = 0; t < L; t += p.tile_queries) {
        const double nq = std::min(p.tile_queries, L - t), qpos = ctx - L + t;
        tile_keys += qpos + nq;
        pf_flops += 4.0 * c.d * G * c.hkv * (nq * qpos + nq * (nq + 1) / 2.0);
      }
    }
    for (int i = 0; i < b->num_decode; ++i)
      dc_bytes += (double)b->decode_ctx_len[i] * kv_tok_bytes + qo_row_bytes + page_bytes * ceil_div(b->decode_ctx_len[i], kPage);
    const bool prefill_heavy = pf_flops / kPrefillFlopsPerSec >= kPrefillHeavyRatio * dc_bytes / kDecodeBytesPerSec;
    if (dc_bytes > 0.0 && !prefill_heavy && (c.mode == POD_ATTN_MODE_FUSED || c.mode == POD_ATTN_MODE_STREAMS))
      beside_split = tile_keys * c.hkv / num_cus;
  }
  for (int i = 0; i < b->num_prefill; ++i) {
    const int L = b->prefill_q_start[i + 1] - b->prefill_q_start[i];
    const int ctx = b->prefill_ctx_len[i];
    if (L == 0) continue;
    if (is_small(L)) { small_chunks.push_back(i); continue; }
    p.prefill_bytes += (double)ctx * kv_tok_bytes + (double)L * qo_row_bytes + page_bytes * ceil_div(ctx, kPage);
    int ns_c = std::max(1, std::min(std::min(cap, kMaxCombineSplits), ceil_div(ctx, kMinPrefillSplit)));
    if (beside_split > kMinPrefillSplit)       // pieces of about beside_split keys (rounded)
      ns_c = std::max(1, std::min(ns_c, (int)std::lround(ctx / beside_split)));
    const int st = round_up_int(ceil_div(ctx, ns_c), kPrefillKvTile);
    ns_c = ceil_div(ctx, st);
    std::vector<Tile> tiles;
    for (int t = 0; t < L; t += p.tile_queries) {
      Tile tl;
      tl.seq = i;
      tl.q_row = b->prefill_q_start[i] + t;
      tl.n_q = std::min(p.tile_queries, L - t);
      tl.q_pos = ctx - L + t;
      tl.kv_len = tl.q_pos + tl.n_q;
      tiles.push_back(tl);
    }
    std::reverse(tiles.begin(), tiles.end());  // last (longest) tile first
    const size_t g0 = pgroups.size();
    pgroups.resize(g0 + (size_t)ns_c * c.hkv);
    for (const Tile& tl : tiles) {
      const int ns = ceil_div(tl.kv_len, st);
      const int di = (int)(p.pdesc.size() / kDescInts);
      std::vector<int32_t> d(kDescInts, 0);
      d[kDSeq] = tl.seq; d[kDQRow] = tl.q_row; d[kDNq] = tl.n_q; d[kDQPos] = tl.q_pos;
      d[kDKvLen] = tl.kv_len; d[kDNSplit] = ns; d[kDSplitTok] = st;
      d[kDGroupBegin] = group; d[kDPartBase] = slot; d[kDNcols] = tl.n_q * G;
      if (ns > 1) { group += c.hkv; slot += c.hkv * ns * tl.n_q * G; }
      p.prefill_max_splits = std::max(p.prefill_max_splits, ns);
      p.prefill_flops += 4.0 * c.d * G * c.hkv *
                         ((double)tl.n_q * tl.q_pos + (double)tl.n_q * (tl.n_q + 1) / 2.0);
      p.pdesc.insert(p.pdesc.end(), d.begin(), d.end());
      for (int sp = 0; sp < ns; ++sp) {
        const double keys = std::min(tl.kv_len, (sp + 1) * st) - sp * st;
        for (int h = 0; h < c.hkv; ++h) {
          PGroup& pg = pgroups[g0 + (size_t)sp * c.hkv + h];
          pg.work += keys * tl.n_q;
          pg.items.push_back(di);
          pg.items.push_back((sp << 16) | h);
        }
      }
    }
  }
  p.n_pdesc = (int)(p.pdesc.size() / kDescInts);
  std::vector<int> gorder(pgroups.size());
  std::iota(gorder.begin(), gorder.end(), 0);
  std::stable_sort(gorder.begin(), gorder.end(), [&](int x, int y) { return pgroups[x].work > pgroups[y].work; });
  std::vector<int32_t> per_xcd[kXcds];
  double load[kXcds] = {0};
  for (int gi : gorder) {
    if (pgroups[gi].items.empty()) continue;
    const int x = (int)(std::min_element(load, load + kXcds) - load);
    load[x] += pgroups[gi].work;
    per_xcd[x].insert(per_xcd[x].end(), pgroups[gi].items.begin(), pgroups[gi].items.end());
  }
  p.pitems.assign(kPItemHeader, 0);
  for (int x = 0; x < kXcds; ++x) {
    p.pitems[x] = (int32_t)((p.pitems.size() - kPItemHeader) / 2);
    p.pitems.insert(p.pitems.end(), per_xcd[x].begin(), per_xcd[x].end());
  }
  p.n_pf_items = (int)((p.pitems.size() - kPItemHeader) / 2);
  p.pitems[kXcds] = p.n_pf_items;
  p.n_pf_groups = group;

  // ---------------- decode sequences and small-q extend pieces
  struct DPiece { int seq, q_row, n_q, q_pos, kv_len; };   // a decode, or a small-q extend chunk
  std::vector<DPiece> pieces;
  for (int i = 0; i < b->num_decode; ++i)
    pieces.push_back({b->num_prefill + i, (int)prefill_rows + i, 1, b->decode_ctx_len[i] - 1, b->decode_ctx_len[i]});
  for (int i : small_chunks) {
    const int L = b->prefill_q_start[i + 1] - b->prefill_q_start[i];
    const int ctx = b->prefill_ctx_len[i];
    pieces.push_back({i, b->prefill_q_start[i], L, ctx - L, ctx});
  }
  for (const DPiece& pc : pieces)   // every piece is a whole sequence's rows: its context once
    p.decode_bytes += (double)pc.kv_len * kv_tok_bytes + (double)pc.n_q * qo_row_bytes + page_bytes * ceil_div(pc.kv_len, kPage);
  p.num_small_extends = (int)small_chunks.size();
  long total_tok = 0;
  for (const DPiece& pc : pieces) total_tok += (long)pc.kv_len * c.hkv;
  int st_target;
  bool one_round = false;                       // prefill-heavy fused plan: decode items start at once
  if (c.decode_split_tokens > 0) {
    st_target = c.decode_split_tokens;
  } else {
    // About one item per decode wave of the grid: fewer, longer items cost fewer partials,
    // tickets and combine work, and the tapered tail below keeps the end of the queue short.
    // Measured, fused kernel us, one / two / three items per wave: Llama-2-7B-shaped 679 / 690 /
    // 705, Llama-3-8B-shaped 1617 / 1616 / 1615, long-context 5040 / 5060 / 5094, speculative
    // verification 1696 / 1701; separate mode on the first 740 / 757.
    // Streams handles keep two per wave: their decode kernel shares the GPU with a concurrent
    // prefill kernel, and one long item per wave left a tail there (long-context batch 5549 ->
    // 6120 us, Llama-2-7B-shaped 730 -> 756 us).
    const int per_wave = c.decode_items_per_wave > 0 ? c.decode_items_per_wave
                                                     : (c.mode == POD_ATTN_MODE_STREAMS ? 2 : 1);
    long target_items = (long)num_cus * wgs_per_cu * kWaves * per_wave;
    // Fused handles, when the prefill share is about as long as the decode share: about one
    // item per workgroup slot instead.  The decode-role workgroups that find the queue empty
    // take prefill tiles, so the matrix work gets the CUs the stream does not need (measured on
    // the Yi-6B-shaped batch: 601 -> 574 us; decode-dominant batches keep the rule above, where
    // it was measured best).  Shares estimated at what the tile and the stream sustain.  The
    // separate decode kernel keeps many items (one workgroup per four).
    const double t_prefill = p.prefill_flops / kPrefillFlopsPerSec, t_decode = p.decode_bytes / kDecodeBytesPerSec;
    if (c.mode == POD_ATTN_MODE_FUSED && t_prefill >= kPrefillHeavyRatio * t_decode) {
      target_items = (long)num_cus * wgs_per_cu;
      one_round = true;
    }
    long st = (total_tok + target_items - 1) / std::max(1L, target_items);
    // The same token count for every cache: an FP8 item streams half the bytes of a bf16 one,
    // but doubling its tokens to make it last as long halves the number of items, and a batch
    // whose items are not already capped by their sequences then leaves half the decode waves
    // idle (FP8 decode-only batches at Llama-3-8B heads, fused kernel us, doubled -> not:
    // 32 x 4K 98.9 -> 67.9, 128 x 32K 2558 -> 1406; the Llama-2-7B-, Llama-3-8B-shaped and
    // long-context FP8 batches within 0.5% fused, the Llama-3-8B-shaped one 1624 -> 1548
    // separate).
    // The one-item-per-slot plan stops at 8192 tokens (5120 with an FP8 cache): the longest
    // items end the launch (Yi-6B-shaped batch, fused kernel us, bf16 cap 8192 / 6144 / 5120:
    // 540.9 / 546.7 / 553.6; FP8 cap 8192 / 6144 / 5120 / 4096: 579.8 / 561.2 / 544.5 / 571.7,
    // and the FP8 Llama-3-8B-shaped batch 1248.8 / 1230.6 / 1250.5 / 1249.7; earlier, that FP8
    // batch: 32768-token items 1503 us, 16384: 1347).
    if (one_round)
      st = std::min(st, (long)(c.dtype == POD_ATTN_FP8_E4M3 ? kOneRoundMaxSplitFp8 : kOneRoundMaxSplit));
    // Floor: a small batch still spreads over the decode waves, down to 256-token items (eight
    // steps; fused kernel us, 512 -> 256 / 128-token floor: 8 decodes at 4K with 4 KV heads
    // 42.5 -> 38.1 / 47.6, 32 at 4K 78.6 -> 72.8 / 71.3, with an FP8 cache 61.9 -> 52.6 / 52.9;
    // 8 at 8K with 8 KV heads 79.4 -> 72.4 / 72.1; larger batches within 1.5%).
    st = std::max((long)kMinDecodeSplit, std::min(32768L, st));
    st_target = round_up_int((int)st, 128);
  }
  p.decode_split_tokens = st_target;
  // Tapered tail: items are claimed in queue order, and when the queue runs dry every wave is
  // still finishing its last item.  When the sequences' lengths vary, the pieces claimed last
  // (about two short items per wave of the grid) take 1/decode_taper of the split length
  // (measured on the Llama-3-8B-shaped batch, 4K-32K contexts: 1692 -> 1640 us).  Batches of
  // equal sequences keep one length: there the extra items' fixed costs (pipeline fill, partial
  // merge) outweighed the shorter tail (Llama-2-7B-shaped batch: 690 -> 704 us).  Not for the
  // one-round plan of a prefill-heavy fused batch, whose decode items all start at once.
  int kv_min = INT32_MAX, kv_max = 0;
  for (const DPiece& pc : pieces) kv_min = std::min(kv_min, pc.kv_len), kv_max = std::max(kv_max, pc.kv_len);
  const bool varied = !pieces.empty() && 2L * kv_max >= 3L * kv_min;
  const int st_tail = std::max(512, round_up_int(st_target / std::max(1, c.decode_taper), 128));
  long tail_tok = 0;
  if (c.decode_taper >= 2 && c.decode_split_tokens == 0 && !one_round && varied && st_tail < st_target)
    tail_tok = std::min(total_tok / 2, 2L * num_cus * wgs_per_cu * kWaves * st_tail);
  std::vector<int> order(pieces.size());
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return pieces[x].kv_len > pieces[y].kv_len; });
  int ditem = 0;
  p.decode_max_splits = 0;
  p.decode_max_cols = G;
  long left_tok = total_tok;                    // key-head tokens of this piece and the ones after it
  for (int i : order) {
    const DPiece& pc = pieces[i];
    const int kv = pc.kv_len, ncols = pc.n_q * G;
    const int st_piece = left_tok <= tail_tok ? st_tail : st_target;
    left_tok -= (long)kv * c.hkv;
    int ns = std::min(kMaxCombineSplits, ceil_div(kv, st_piece));
    int st = round_up_int(ceil_div(kv, ns), 128);
    ns = ceil_div(kv, st);
    std::vector<int32_t> d(kDescInts, 0);
    d[kDSeq] = pc.seq; d[kDQRow] = pc.q_row; d[kDNq] = pc.n_q;
    d[kDQPos] = pc.q_pos; d[kDKvLen] = kv; d[kDNSplit] = ns; d[kDSplitTok] = st;
    d[kDItemBegin] = ditem; d[kDGroupBegin] = group; d[kDPartBase] = slot; d[kDNcols] = ncols;
    ditem += c.hkv * ns;
    if (ns > 1) { group += c.hkv; slot += c.hkv * ns * ncols; }
    p.decode_max_splits = std::max(p.decode_max_splits, ns);
    p.decode_max_cols = std::max(p.decode_max_cols, ncols);
    p.decode_flops += 4.0 * c.d * c.hq * ((double)pc.n_q * pc.q_pos + (double)pc.n_q * (pc.n_q + 1) / 2.0);
    p.ddesc.insert(p.ddesc.end(), d.begin(), d.end());
  }
  p.n_ddesc = (int)pieces.size();
  p.n_dc_items = ditem;
  p.n_groups = group;
  p.n_slots = slot;

  // ---------------- workspace map
  WorkspaceMap m{};
  size_t off = 0;
  m.ctrl = off; off = align_up(off + sizeof(int32_t) * kCtrlInts, 256);
  m.tickets = off; off = align_up(off + sizeof(int32_t) * std::max(1, p.n_groups), 256);
  m.claims = off;
  if (c.flags & POD_ATTN_FLAG_DEBUG_CLAIMS)
    off = align_up(off + sizeof(int32_t) * std::max(1, p.n_pf_items + p.n_dc_items), 256);
  m.pdesc = off; off = align_up(off + sizeof(int32_t) * std::max<size_t>(1, p.pdesc.size()), 256);
  m.pitems = off; off = align_up(off + sizeof(int32_t) * p.pitems.size(), 256);
  m.ddesc = off; off = align_up(off + sizeof(int32_t) * std::max<size_t>(1, p.ddesc.size()), 256);
  m.aunits = off; off = align_up(off + sizeof(int32_t) * std::max<size_t>(1, p.aunits.size()), 256);
  m.copy_bytes = off;
  m.part_o = off; off = align_up(off + sizeof(float) * (size_t)p.n_slots * c.d, 256);
  m.part_lse = off; off = align_up(off + sizeof(float) * (size_t)std::max(1, p.n_slots), 256);
  m.trace = off;
  if (c.flags & POD_ATTN_FLAG_TRACE)
    off = align_up(off + 4 * sizeof(uint32_t) * (size_t)std::max(1, p.n_pf_items + p.n_dc_items), 256);
  m.total = off;
  p.map = m;
  *out = std::move(p);
  return POD_ATTN_OK;
}

void stage_plan(const Plan& p, const Config& c, uint8_t* dst, bool with_units) {
  const size_t base = p.map.pdesc;             // [0, pdesc) is zero-filled on the device
  std::memset(dst, 0, (with_units ? p.map.copy_bytes : p.map.aunits) - base);
  if (!p.pdesc.empty()) std::memcpy(dst + p.map.pdesc - base, p.pdesc.data(), p.pdesc.size() * 4);
  std::memcpy(dst + p.map.pitems - base, p.pitems.data(), p.pitems.size() * 4);
  if (!p.ddesc.empty()) std::memcpy(dst + p.map.ddesc - base, p.ddesc.data(), p.ddesc.size() * 4);
  if (with_units && !p.aunits.empty()) std::memcpy(dst + p.map.aunits - base, p.aunits.data(), p.aunits.size() * 4);
  (void)c;
}

void expand_items(const Plan& p, const Config& c, std::vector<int32_t>* items) {
  items->clear();
  const int G = c.group();
  auto emit = [&](const int32_t* d, int s, int h, int kind, int queue) {
    const int ns = d[kDNSplit], st = d[kDSplitTok];
    int32_t it[16] = {0};
    it[0] = d[kDSeq]; it[1] = d[kDQRow]; it[2] = d[kDNq]; it[3] = d[kDQPos];
    it[4] = h; it[5] = s * st; it[6] = std::min(d[kDKvLen], (s + 1) * st);
    it[7] = ns > 1 ? d[kDGroupBegin] + h : -1;
    it[8] = s;
    it[9] = ns > 1 ? d[kDPartBase] + (h * ns + s) * d[kDNq] * G : -1;
    it[10] = kind;
    it[11] = queue;
    items->insert(items->end(), it, it + 16);
  };
  // prefill: in item-table order (the per-XCD queues back to back)
  int queue = 0;
  for (int i = 0; i < p.n_pf_items; ++i) {
    while (queue + 1 < kXcds && i >= p.pitems[queue + 1]) ++queue;
    const int32_t* e = &p.pitems[kPItemHeader + 2 * (size_t)i];
    emit(&p.pdesc[(size_t)e[0] * kDescInts], e[1] >> 16, e[1] & 0xFFFF, 0, queue);
  }
  // decode: descriptor order, split-major, as the kernels decode items
  for (int di = 0; di < p.n_ddesc; ++di) {
    const int32_t* d = &p.ddesc[(size_t)di * kDescInts];
    for (int s = 0; s < d[kDNSplit]; ++s)
      for (int h = 0; h < c.hkv; ++h) emit(d, s, h, 1, -1);
  }
}

}  // namespace pod

/*
 * pkv_oracle.c -- plain, slow, fp64 CPU oracle for paged-KV decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this file's library.  The GPU product
 * path never calls it, and this file shares no code, header or constant with
 * the HIP library.
 *
 * What it computes (plain definitions, no blocking, no fusion):
 *
 *  - The paged KV cache is one contiguous array of bf16 values laid out
 *    [num_layers, num_pages, 2, page_size, num_kv_heads, head_dim]; index 0 of
 *    the third axis holds keys, index 1 holds values ("Adding a Model",
 *    vox-serve docs, section 1 "The model code").
 *  - A request's pages are listed in a CSR page table (page_indptr,
 *    page_indices) with last_page_len = rows used in its final page, counted
 *    after this step's row is appended.  The pages only say that the runtime
 *    writes "KV page tables" each step ("Adding a Model", "How a program
 *    runs"); the CSR encoding is the reading this oracle takes.
 *  - Token t of a request sits in page page_indices[page_indptr[b] + t / PS],
 *    slot t % PS; the request holds L = (n - 1) * PS + last_page_len tokens.
 *  - Append ("set_kv_cache(kv_cache, k, v)" in section 1 of "Adding a
 *    Model"): copy each entry's new K and V rows, bit for bit, into slot
 *    last_page_len - 1 of its last listed page.  Padding entries list scratch
 *    page 0 ("How a program runs": unused entries point at KV page 0).
 *  - Decode ("run(q, kv_cache)", one query row per request): for query head
 *    hq, KV head h = hq / (Hq / Hkv) (contiguous GQA groups), scores
 *    s_t = sm_scale * <q, K_t>, weights w_t = exp(s_t - lse) with
 *    lse = ln(sum_t exp(s_t)), out = sum_t w_t V_t.  lse is a natural log.
 *  - Split mode: the same over fixed runs of chunk_pages pages, giving one
 *    (o_c, lse_c) per run, then the log-sum-exp merge of the partial
 *    attentions ("Supported Models", M* docs, LTX-2.5 notes: queries merge
 *    the ranks' partial attentions).
 *
 *  - Paged prefill and mixed steps ("Adding a Model", "How a program runs":
 *    prefill runs several rows per request over the same paged cache;
 *    "Supported Models", Qwen3-Omni / Qwen3-TTS notes: new prompts ride a
 *    decode step as a mixed step).  Entry b brings n_b = qo_indptr[b+1] -
 *    qo_indptr[b] new rows (n_b = 1 is a decode row); after they are
 *    appended its L tokens end with them, at positions L - n_b .. L - 1.
 *    Row j of entry b sits at position p = L - n_b + j and attends tokens
 *    0 .. p (causal), with the decode formula above.
 *  - Fused q/k norm, rotary embedding and KV write ("Supported Models", M*
 *    docs, Qwen3-Omni and Qwen3-TTS notes: each layer's q/k RMSNorm, RoPE and
 *    KV write run as one kernel, in fp32 throughout and rounded once, with
 *    the RoPE theta taken from the position resource).  Per head of D values
 *    x: y = x / sqrt(mean(x^2) + eps) * w (RMSNorm over the head, weight w of
 *    D values, one for q heads and one for k heads); then the rotary
 *    embedding at the entry's position p in the rotate-half pairing of
 *    Qwen3-style attention: for i < D/2, with angle a_i = p * theta^(-2i/D),
 *      z_i       = y_i cos a_i - y_{i+D/2} sin a_i
 *      z_{i+D/2} = y_{i+D/2} cos a_i + y_i sin a_i.
 *    The rotated q rows are returned; the rotated k rows (rounded to bf16)
 *    and the v rows (bit copies) go to the slot the append fills.  The
 *    pages name the fusion but not its formulas: the RMSNorm and the
 *    rotate-half pairing are the readings this oracle takes.
 *
 * All arithmetic is fp64; every bf16 input is widened exactly.
 * Functions return 0 on success and a negative value on a malformed table.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Exact bf16 -> fp64 widening: a bf16 value is the top half of an fp32. */
static double widen_bf16(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/*
 * Round an fp64 value to the nearest bf16 (ties to even), directly: a bf16 is
 * the top 16 bits of an fp32, so first round to fp32, then to bf16, and where
 * the fp32 lands exactly halfway between two bf16 values although the fp64
 * value did not, round toward the fp64 value instead of to even.  Finite
 * inputs only.
 */
uint16_t oracle_bf16_round(double x)
{
    float f = (float)x;
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0xFFFFu) == 0x8000u && (double)f != x) {
        uint32_t hi = u >> 16;   /* the bf16 below f in magnitude */
        return (uint16_t)(fabs(x) > fabs((double)f) ? hi + 1 : hi);
    }
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* Element index of cache[layer][page][kv][slot][head][0]. */
static int64_t cache_row(int64_t num_pages, int64_t page_size, int64_t num_kv_heads,
                         int64_t head_dim, int64_t layer, int64_t page, int64_t kv,
                         int64_t slot, int64_t head)
{
    int64_t r = layer;
    r = r * num_pages + page;
    r = r * 2 + kv;
    r = r * page_size + slot;
    r = r * num_kv_heads + head;
    return r * head_dim;
}

/* Number of tokens entry b holds, or -1 if its table row is malformed. */
static int64_t entry_len(const int32_t *indptr, const int32_t *last_len,
                         int64_t page_size, int64_t b)
{
    int64_t n = (int64_t)indptr[b + 1] - (int64_t)indptr[b];
    if (n < 1 || last_len[b] < 1 || last_len[b] > page_size)
        return -1;
    return (n - 1) * page_size + last_len[b];
}

int oracle_append(uint16_t *cache, int64_t num_layers, int64_t num_pages,
                  int64_t page_size, int64_t num_kv_heads, int64_t head_dim,
                  int64_t layer, const uint16_t *k_new, const uint16_t *v_new,
                  const int32_t *page_indptr, const int32_t *page_indices,
                  const int32_t *last_page_len, int64_t batch)
{
    if (layer < 0 || layer >= num_layers)
        return -1;
    for (int64_t b = 0; b < batch; ++b) {
        if (entry_len(page_indptr, last_page_len, page_size, b) < 0)
            return -2;
        int64_t page = page_indices[page_indptr[b + 1] - 1];
        int64_t slot = last_page_len[b] - 1;
        if (page < 0 || page >= num_pages)
            return -3;
        for (int64_t h = 0; h < num_kv_heads; ++h) {
            int64_t src = (b * num_kv_heads + h) * head_dim;
            int64_t dk = cache_row(num_pages, page_size, num_kv_heads, head_dim,
                                   layer, page, 0, slot, h);
            int64_t dv = cache_row(num_pages, page_size, num_kv_heads, head_dim,
                                   layer, page, 1, slot, h);
            for (int64_t d = 0; d < head_dim; ++d) {
                cache[dk + d] = k_new[src + d];
                cache[dv + d] = v_new[src + d];
            }
        }
    }
    return 0;
}

/*
 * Attention of one query row over tokens [t0, t1) of entry b, KV head h.
 * Writes o[head_dim] and *lse.  scores is caller scratch of >= t1 - t0.
 */
static void attend_range(const uint16_t *cache, int64_t num_pages, int64_t page_size,
                         int64_t num_kv_heads, int64_t head_dim, int64_t layer,
                         const uint16_t *qrow, int64_t h, const int32_t *pages,
                         int64_t t0, int64_t t1, double sm_scale, double *scores,
                         double *o, double *lse)
{
    /* scores */
    double m = -INFINITY;
    for (int64_t t = t0; t < t1; ++t) {
        int64_t page = pages[t / page_size];
        int64_t kr = cache_row(num_pages, page_size, num_kv_heads, head_dim, layer,
                               page, 0, t % page_size, h);
        double dot = 0.0;
        for (int64_t d = 0; d < head_dim; ++d)
            dot += widen_bf16(qrow[d]) * widen_bf16(cache[kr + d]);
        scores[t - t0] = sm_scale * dot;
        if (scores[t - t0] > m)
            m = scores[t - t0];
    }
    /* log-sum-exp, shifted by the max so exp never overflows */
    double z = 0.0;
    for (int64_t t = t0; t < t1; ++t)
        z += exp(scores[t - t0] - m);
    *lse = m + log(z);
    /* weighted sum of value rows */
    for (int64_t d = 0; d < head_dim; ++d)
        o[d] = 0.0;
    for (int64_t t = t0; t < t1; ++t) {
        int64_t page = pages[t / page_size];
        int64_t vr = cache_row(num_pages, page_size, num_kv_heads, head_dim, layer,
                               page, 1, t % page_size, h);
        double w = exp(scores[t - t0] - *lse);
        for (int64_t d = 0; d < head_dim; ++d)
            o[d] += w * widen_bf16(cache[vr + d]);
    }
}

/* One (entry, query head) row, unsplit (chunk_pages <= 0) or split + merged. */
static int decode_row(const uint16_t *cache, int64_t num_pages, int64_t page_size,
                      int64_t num_kv_heads, int64_t head_dim, int64_t layer,
                      const uint16_t *q, int64_t num_qo_heads,
                      const int32_t *page_indptr, const int32_t *page_indices,
                      const int32_t *last_page_len, int64_t b, int64_t hq,
                      double sm_scale, int64_t chunk_pages, double *out, double *lse)
{
    int64_t len = entry_len(page_indptr, last_page_len, page_size, b);
    if (len < 0)
        return -2;
    const int32_t *pages = page_indices + page_indptr[b];
    int64_t npages = page_indptr[b + 1] - page_indptr[b];
    for (int64_t i = 0; i < npages; ++i)
        if (pages[i] < 0 || pages[i] >= num_pages)
            return -3;
    int64_t group = num_qo_heads / num_kv_heads;
    int64_t h = hq / group;
    const uint16_t *qrow = q + (b * num_qo_heads + hq) * head_dim;

    double *scores = malloc(sizeof(double) * (size_t)len);
    if (!scores)
        return -4;
    if (chunk_pages <= 0) {
        attend_range(cache, num_pages, page_size, num_kv_heads, head_dim, layer, qrow,
                     h, pages, 0, len, sm_scale, scores, out, lse);
        free(scores);
        return 0;
    }

    /* Split mode: partial (o_c, lse_c) per run of chunk_pages pages ... */
    int64_t chunk_tokens = chunk_pages * page_size;
    int64_t nchunks = (len + chunk_tokens - 1) / chunk_tokens;
    double *o_c = malloc(sizeof(double) * (size_t)(nchunks * head_dim));
    double *lse_c = malloc(sizeof(double) * (size_t)nchunks);
    if (!o_c || !lse_c) {
        free(scores);
        free(o_c);
        free(lse_c);
        return -4;
    }
    for (int64_t c = 0; c < nchunks; ++c) {
        int64_t t0 = c * chunk_tokens;
        int64_t t1 = t0 + chunk_tokens < len ? t0 + chunk_tokens : len;
        attend_range(cache, num_pages, page_size, num_kv_heads, head_dim, layer, qrow,
                     h, pages, t0, t1, sm_scale, scores, o_c + c * head_dim, &lse_c[c]);
    }
    /* ... then the log-sum-exp merge of the partials. */
    double mx = -INFINITY;
    for (int64_t c = 0; c < nchunks; ++c)
        if (lse_c[c] > mx)
            mx = lse_c[c];
    double s = 0.0;
    for (int64_t c = 0; c < nchunks; ++c)
        s += exp(lse_c[c] - mx);
    *lse = mx + log(s);
    for (int64_t d = 0; d < head_dim; ++d)
        out[d] = 0.0;
    for (int64_t c = 0; c < nchunks; ++c) {
        double w = exp(lse_c[c] - *lse);
        for (int64_t d = 0; d < head_dim; ++d)
            out[d] += w * o_c[c * head_dim + d];
    }
    free(o_c);
    free(lse_c);
    free(scores);
    return 0;
}

/*
 * Decode every (entry, query head) row.  out is fp64 [batch, Hq, head_dim],
 * lse is fp64 [batch, Hq].  chunk_pages <= 0 means unsplit.
 */
int oracle_decode(const uint16_t *cache, int64_t num_layers, int64_t num_pages,
                  int64_t page_size, int64_t num_kv_heads, int64_t head_dim,
                  int64_t layer, const uint16_t *q, int64_t num_qo_heads,
                  const int32_t *page_indptr, const int32_t *page_indices,
                  const int32_t *last_page_len, int64_t batch, double sm_scale,
                  int64_t chunk_pages, double *out, double *lse)
{
    if (layer < 0 || layer >= num_layers || num_kv_heads < 1 ||
        num_qo_heads % num_kv_heads != 0)
        return -1;
    for (int64_t b = 0; b < batch; ++b)
        for (int64_t hq = 0; hq < num_qo_heads; ++hq) {
            int rc = decode_row(cache, num_pages, page_size, num_kv_heads, head_dim,
                                layer, q, num_qo_heads, page_indptr, page_indices,
                                last_page_len, b, hq, sm_scale, chunk_pages,
                                out + (b * num_qo_heads + hq) * head_dim,
                                lse + b * num_qo_heads + hq);
            if (rc)
                return rc;
        }
    return 0;
}

/*
 * Decode a chosen list of rows (row_b[i], row_hq[i]), for spot checks of large
 * batches.  out is fp64 [nrows, head_dim], lse is fp64 [nrows].
 */
int oracle_decode_rows(const uint16_t *cache, int64_t num_layers, int64_t num_pages,
                       int64_t page_size, int64_t num_kv_heads, int64_t head_dim,
                       int64_t layer, const uint16_t *q, int64_t num_qo_heads,
                       const int32_t *page_indptr, const int32_t *page_indices,
                       const int32_t *last_page_len, int64_t batch, double sm_scale,
                       int64_t chunk_pages, const int64_t *row_b, const int64_t *row_hq,
                       int64_t nrows, double *out, double *lse)
{
    if (layer < 0 || layer >= num_layers || num_kv_heads < 1 ||
        num_qo_heads % num_kv_heads != 0)
        return -1;
    for (int64_t i = 0; i < nrows; ++i) {
        if (row_b[i] < 0 || row_b[i] >= batch || row_hq[i] < 0 ||
            row_hq[i] >= num_qo_heads)
            return -1;
        int rc = decode_row(cache, num_pages, page_size, num_kv_heads, head_dim, layer,
                            q, num_qo_heads, page_indptr, page_indices, last_page_len,
                            row_b[i], row_hq[i], sm_scale, chunk_pages,
                            out + i * head_dim, lse + i);
        if (rc)
            return rc;
    }
    return 0;
}

/* RMSNorm of one head row: y = x / sqrt(mean(x^2) + eps) * w. */
static void rms_norm_row(const uint16_t *x, const uint16_t *w, int64_t head_dim,
                         double eps, double *y)
{
    double ss = 0.0;
    for (int64_t d = 0; d < head_dim; ++d) {
        double v = widen_bf16(x[d]);
        ss += v * v;
    }
    double inv = 1.0 / sqrt(ss / (double)head_dim + eps);
    for (int64_t d = 0; d < head_dim; ++d)
        y[d] = widen_bf16(x[d]) * inv * widen_bf16(w[d]);
}

/* Rotary embedding of one head row in place, rotate-half pairing: element i
 * and element i + D/2 turn by the angle pair_pos[i] * theta^(-2i/D), where
 * pair_pos[i] is the position pair i follows (the entry's position for plain
 * RoPE; for multimodal RoPE the component of the entry's (t, h, w) position
 * named for that pair). */
static void rope_row(double *y, int64_t head_dim, const double *pair_pos, double theta)
{
    int64_t half = head_dim / 2;
    for (int64_t i = 0; i < half; ++i) {
        double angle = pair_pos[i] * pow(theta, -2.0 * (double)i / (double)head_dim);
        double c = cos(angle), s = sin(angle);
        double lo = y[i], hi = y[i + half];
        y[i] = lo * c - hi * s;
        y[i + half] = hi * c + lo * s;
    }
}

/*
 * The q/k norm, rotary embedding and KV write of one layer, for plain RoPE
 * (pos_stride 1, pair_axis NULL: every pair follows positions[b]) and for
 * multimodal RoPE (pos_stride 3: positions[b] is the entry's (t, h, w)
 * position, and pair i follows component pair_axis[i]).
 */
static int norm_rope_append(uint16_t *cache, int64_t num_layers, int64_t num_pages,
                            int64_t page_size, int64_t num_kv_heads, int64_t head_dim,
                            int64_t layer, const uint16_t *q, int64_t num_qo_heads,
                            const uint16_t *k_new, const uint16_t *v_new,
                            const uint16_t *q_w, const uint16_t *k_w, double eps,
                            double theta, const int32_t *positions, int64_t pos_stride,
                            const uint8_t *pair_axis, const int32_t *page_indptr,
                            const int32_t *page_indices, const int32_t *last_page_len,
                            int64_t batch, double *q_out, double *k_out)
{
    if (layer < 0 || layer >= num_layers || head_dim % 2 != 0 || head_dim > 512)
        return -1;
    double pair_pos[256];
    for (int64_t b = 0; b < batch; ++b) {
        if (entry_len(page_indptr, last_page_len, page_size, b) < 0)
            return -2;
        int64_t page = page_indices[page_indptr[b + 1] - 1];
        int64_t slot = last_page_len[b] - 1;
        if (page < 0 || page >= num_pages)
            return -3;
        for (int64_t i = 0; i < head_dim / 2; ++i) {
            int64_t axis = pair_axis ? pair_axis[i] : 0;
            if (axis < 0 || axis >= pos_stride)
                return -4;
            pair_pos[i] = (double)positions[b * pos_stride + axis];
        }
        for (int64_t hq = 0; hq < num_qo_heads; ++hq) {
            int64_t row = (b * num_qo_heads + hq) * head_dim;
            rms_norm_row(q + row, q_w, head_dim, eps, q_out + row);
            rope_row(q_out + row, head_dim, pair_pos, theta);
        }
        for (int64_t h = 0; h < num_kv_heads; ++h) {
            int64_t row = (b * num_kv_heads + h) * head_dim;
            rms_norm_row(k_new + row, k_w, head_dim, eps, k_out + row);
            rope_row(k_out + row, head_dim, pair_pos, theta);
            int64_t dk = cache_row(num_pages, page_size, num_kv_heads, head_dim,
                                   layer, page, 0, slot, h);
            int64_t dv = cache_row(num_pages, page_size, num_kv_heads, head_dim,
                                   layer, page, 1, slot, h);
            for (int64_t d = 0; d < head_dim; ++d) {
                cache[dk + d] = oracle_bf16_round(k_out[row + d]);
                cache[dv + d] = v_new[row + d];
            }
        }
    }
    return 0;
}

/*
 * q_out[b, hq, :] = rope(rmsnorm(q[b, hq, :], q_w), positions[b]) (fp64), and
 * k_out[b, h, :] = rope(rmsnorm(k_new[b, h, :], k_w), positions[b]) (fp64),
 * whose bf16 rounding goes to the K slot the append fills, with v_new[b, h, :]
 * copied bit for bit to the V slot (same page and slot as oracle_append).
 * head_dim must be even.
 */
int oracle_qk_norm_rope_append(uint16_t *cache, int64_t num_layers, int64_t num_pages,
                               int64_t page_size, int64_t num_kv_heads, int64_t head_dim,
                               int64_t layer, const uint16_t *q, int64_t num_qo_heads,
                               const uint16_t *k_new, const uint16_t *v_new,
                               const uint16_t *q_w, const uint16_t *k_w, double eps,
                               double theta, const int32_t *positions,
                               const int32_t *page_indptr, const int32_t *page_indices,
                               const int32_t *last_page_len, int64_t batch,
                               double *q_out, double *k_out)
{
    return norm_rope_append(cache, num_layers, num_pages, page_size, num_kv_heads, head_dim,
                            layer, q, num_qo_heads, k_new, v_new, q_w, k_w, eps, theta,
                            positions, 1, NULL, page_indptr, page_indices, last_page_len,
                            batch, q_out, k_out);
}

/*
 * The same with multimodal RoPE: positions is [batch, 3], the (t, h, w)
 * position of each entry's new token, and rotary pair i (elements i and
 * i + D/2) turns by positions[b, pair_axis[i]] * theta^(-2i/D); pair_axis
 * holds D/2 entries, each 0, 1 or 2.  With equal components it is the plain
 * RoPE above.
 */
int oracle_qk_norm_mrope_append(uint16_t *cache, int64_t num_layers, int64_t num_pages,
                                int64_t page_size, int64_t num_kv_heads, int64_t head_dim,
                                int64_t layer, const uint16_t *q, int64_t num_qo_heads,
                                const uint16_t *k_new, const uint16_t *v_new,
                                const uint16_t *q_w, const uint16_t *k_w, double eps,
                                double theta, const int32_t *positions,
                                const uint8_t *pair_axis, const int32_t *page_indptr,
                                const int32_t *page_indices, const int32_t *last_page_len,
                                int64_t batch, double *q_out, double *k_out)
{
    return norm_rope_append(cache, num_layers, num_pages, page_size, num_kv_heads, head_dim,
                            layer, q, num_qo_heads, k_new, v_new, q_w, k_w, eps, theta,
                            positions, 3, pair_axis, page_indptr, page_indices,
                            last_page_len, batch, q_out, k_out);
}

/*
 * Append of several rows per entry: row j of entry b (global row
 * qo_indptr[b] + j) goes to token position L - n_b + j, i.e. page
 * page_indices[page_indptr[b] + t / page_size], slot t % page_size.
 * k_new, v_new: [total rows, num_kv_heads, head_dim].
 */
int oracle_append_rows(uint16_t *cache, int64_t num_layers, int64_t num_pages,
                       int64_t page_size, int64_t num_kv_heads, int64_t head_dim,
                       int64_t layer, const uint16_t *k_new, const uint16_t *v_new,
                       const int32_t *qo_indptr, const int32_t *page_indptr,
                       const int32_t *page_indices, const int32_t *last_page_len,
                       int64_t batch)
{
    if (layer < 0 || layer >= num_layers)
        return -1;
    for (int64_t b = 0; b < batch; ++b) {
        int64_t len = entry_len(page_indptr, last_page_len, page_size, b);
        int64_t n = (int64_t)qo_indptr[b + 1] - (int64_t)qo_indptr[b];
        if (len < 0 || n < 0 || n > len)
            return -2;
        for (int64_t j = 0; j < n; ++j) {
            int64_t t = len - n + j;
            int64_t page = page_indices[page_indptr[b] + t / page_size];
            if (page < 0 || page >= num_pages)
                return -3;
            for (int64_t h = 0; h < num_kv_heads; ++h) {
                int64_t src = ((qo_indptr[b] + j) * num_kv_heads + h) * head_dim;
                int64_t dk = cache_row(num_pages, page_size, num_kv_heads, head_dim,
                                       layer, page, 0, t % page_size, h);
                int64_t dv = cache_row(num_pages, page_size, num_kv_heads, head_dim,
                                       layer, page, 1, t % page_size, h);
                for (int64_t d = 0; d < head_dim; ++d) {
                    cache[dk + d] = k_new[src + d];
                    cache[dv + d] = v_new[src + d];
                }
            }
        }
    }
    return 0;
}

/*
 * Causal attention of every new row: row j of entry b at position
 * p = L - n_b + j over tokens 0 .. p of its pages.  q, out: [total rows,
 * num_qo_heads, head_dim] (out fp64); lse: fp64 [total rows, num_qo_heads].
 */
int oracle_prefill(const uint16_t *cache, int64_t num_layers, int64_t num_pages,
                   int64_t page_size, int64_t num_kv_heads, int64_t head_dim,
                   int64_t layer, const uint16_t *q, int64_t num_qo_heads,
                   const int32_t *qo_indptr, const int32_t *page_indptr,
                   const int32_t *page_indices, const int32_t *last_page_len,
                   int64_t batch, double sm_scale, double *out, double *lse)
{
    if (layer < 0 || layer >= num_layers || num_qo_heads % num_kv_heads != 0)
        return -1;
    int64_t group = num_qo_heads / num_kv_heads;
    for (int64_t b = 0; b < batch; ++b) {
        int64_t len = entry_len(page_indptr, last_page_len, page_size, b);
        int64_t n = (int64_t)qo_indptr[b + 1] - (int64_t)qo_indptr[b];
        if (len < 0 || n < 0 || n > len)
            return -2;
        const int32_t *pages = page_indices + page_indptr[b];
        for (int64_t i = 0; i < page_indptr[b + 1] - page_indptr[b]; ++i)
            if (pages[i] < 0 || pages[i] >= num_pages)
                return -3;
        double *scores = malloc(sizeof(double) * (size_t)len);
        if (!scores)
            return -4;
        for (int64_t j = 0; j < n; ++j) {
            int64_t row = qo_indptr[b] + j;
            int64_t pos = len - n + j;
            for (int64_t hq = 0; hq < num_qo_heads; ++hq) {
                const uint16_t *qrow = q + (row * num_qo_heads + hq) * head_dim;
                attend_range(cache, num_pages, page_size, num_kv_heads, head_dim, layer,
                             qrow, hq / group, pages, 0, pos + 1, sm_scale, scores,
                             out + (row * num_qo_heads + hq) * head_dim,
                             lse + row * num_qo_heads + hq);
            }
        }
        free(scores);
    }
    return 0;
}

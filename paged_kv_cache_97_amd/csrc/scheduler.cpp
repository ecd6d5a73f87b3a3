// Native continuous-batching scheduler (host code; C ABI in include/pkv_sched.h).
//
// The step policy of gaoleia.github.io "PagedAttention 和 Continuous
// Batching" §2.3-§2.6, 5688vip.com "vLLM核心机制" §3.1/§3.3 and
// lakecityint.com/news/209622 §1-§2/§4.2, with the readings the Python
// scheduler of this package takes (request-granular preemption, LIFO victims,
// swapped before waiting, no admission in a step that preempted, decode rows
// before prefill chunks): the two implementations make the same decisions in
// the same order, so their plans are identical.  This one is native because
// planning runs on the host once per step, beside kernels that take tens of
// microseconds.
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <deque>
#include <memory>
#include <string>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "../../include/pagedkv.h"
#include "../../include/pkv_sched.h"

namespace pkv {
int report(int status, const char* msg);  // api.hip
}

namespace {

// Physical block ids handed out first-in first-out, with reference counts.
class BlockPool {
 public:
  void init(int32_t n, const int32_t* order) {
    ref_.assign(n, 0);
    free_.clear();
    for (int32_t i = 0; i < n; ++i) free_.push_back(order ? order[i] : i);
  }
  int32_t num_free() const { return (int32_t)free_.size(); }
  bool alloc(int32_t* b) {
    if (free_.empty()) return false;
    *b = free_.front();
    free_.pop_front();
    ref_[*b] = 1;
    return true;
  }
  void release(int32_t b) {
    if (--ref_[b] == 0) free_.push_back(b);
  }

 private:
  std::deque<int32_t> free_;
  std::vector<int32_t> ref_;
};

enum State { kWaiting = 0, kRunning = 1, kSwapped = 2, kFinished = 3 };

struct Request {
  int64_t id;
  int32_t prompt_len, max_new, arrival;
  int32_t num_computed = 0;
  int32_t recompute_to = 0;
  int32_t num_preemptions = 0;
  State state = kWaiting;
  bool has_table = false;
  std::vector<int32_t> mapping;                       // block table
  int32_t table_tokens = 0;                           // tokens the table holds

  int32_t total_len() const { return prompt_len + max_new; }
  int32_t prefill_target() const { return std::max(prompt_len, recompute_to); }
  bool in_prefill() const { return num_computed < prefill_target(); }
  bool finished() const { return num_computed >= total_len(); }
};

}  // namespace

struct pkv_sched {
  pkv_sched_config cfg;
  BlockPool gpu, cpu;
  std::unordered_map<int64_t, std::unique_ptr<Request>> reqs;
  std::deque<Request*> waiting, swapped;
  std::vector<Request*> running;
  int32_t arrivals = 0;
  int32_t counts[4] = {0, 0, 0, 0};
  bool pending = false;                               // a plan awaits pkv_sched_complete

  // last plan
  std::vector<int64_t> req_id, finished_ids, preempted_ids;
  std::vector<int32_t> start, row_tokens, tables, positions, qsl, seq_lens, swap_out, swap_in;
  std::vector<uint8_t> is_prefill;

  void set_state(Request* r, State st) {
    --counts[r->state];
    r->state = st;
    ++counts[st];
  }
  int32_t blocks_needed(const Request* r, int32_t n) const {
    const int32_t have = r->has_table ? (int32_t)r->mapping.size() : 0;
    const int32_t need = (r->num_computed + n + cfg.block_size - 1) / cfg.block_size;
    return std::max(0, need - have);
  }
  int32_t watermark_blocks() const { return (int32_t)(cfg.watermark * cfg.num_gpu_blocks); }
  int32_t tokens_for(const Request* r, int32_t budget) const {
    if (r->in_prefill())
      return std::min(std::min(cfg.max_prefill_chunk, r->prefill_target() - r->num_computed), budget);
    return std::min(1, budget);
  }
  // Room for n more tokens in r's table (the caller checked the free count).
  void append_tokens(Request* r, int32_t n) {
    const int32_t total = r->table_tokens + n;
    const size_t need = (size_t)((total + cfg.block_size - 1) / cfg.block_size);
    while (r->mapping.size() < need) {
      int32_t b = -1;
      gpu.alloc(&b);
      r->mapping.push_back(b);
    }
    r->table_tokens = total;
  }
  void release_table(Request* r) {
    for (int32_t b : r->mapping) gpu.release(b);
    r->mapping.clear();
    r->table_tokens = 0;
    r->has_table = false;
  }
  void preempt(Request* v) {
    running.erase(std::find(running.begin(), running.end(), v));
    ++v->num_preemptions;
    preempted_ids.push_back(v->id);
    if (cfg.preemption_swap && cpu.num_free() >= (int32_t)v->mapping.size()) {
      for (auto& b : v->mapping) {                    // GPU blocks to CPU blocks
        int32_t c = -1;
        cpu.alloc(&c);
        swap_out.push_back(b);
        swap_out.push_back(c);
        gpu.release(b);
        b = c;
      }
      set_state(v, kSwapped);
      swapped.push_back(v);
      return;
    }
    v->recompute_to = std::max(v->recompute_to, v->num_computed);
    release_table(v);
    v->num_computed = 0;
    set_state(v, kWaiting);
    waiting.push_front(v);
  }

  void schedule() {
    req_id.clear(); start.clear(); row_tokens.clear(); is_prefill.clear(); tables.clear();
    positions.clear(); qsl.clear(); seq_lens.clear(); swap_out.clear(); swap_in.clear();
    finished_ids.clear(); preempted_ids.clear();
    // 1. finished requests leave and free their blocks
    {
      std::vector<Request*> keep;
      keep.reserve(running.size());
      for (Request* r : running) {
        if (r->finished()) {
          release_table(r);
          set_state(r, kFinished);
          finished_ids.push_back(r->id);
        } else {
          keep.push_back(r);
        }
      }
      running.swap(keep);
    }
    int32_t budget_tokens = cfg.max_num_batched_tokens, budget_seqs = cfg.max_num_seqs;
    std::vector<std::pair<Request*, int32_t>> grants;
    // 2. running requests: decodes first, then prefill chunks, each in
    //    admission order; room comes from preempting the newest running ones
    std::vector<Request*> order(running);
    std::stable_sort(order.begin(), order.end(), [](const Request* x, const Request* y) {
      const bool px = x->in_prefill(), py = y->in_prefill();
      if (px != py) return !px;
      return x->arrival < y->arrival;
    });
    std::unordered_set<const Request*> granted;
    for (Request* r : order) {
      if (r->state != kRunning) continue;             // preempted while making room
      if (budget_seqs == 0 || budget_tokens == 0) break;
      const int32_t n = tokens_for(r, budget_tokens);
      const int32_t need = blocks_needed(r, n);
      while (gpu.num_free() < need) {
        Request* victim = nullptr;
        for (Request* v : running)
          if (v != r && !granted.count(v) && (!victim || v->arrival > victim->arrival)) victim = v;
        if (!victim || victim->arrival < r->arrival) victim = r;   // r itself is the newest: it yields
        preempt(victim);
        if (victim == r) break;
      }
      if (r->state != kRunning) continue;
      append_tokens(r, n);
      grants.emplace_back(r, n);
      granted.insert(r);
      budget_tokens -= n;
      --budget_seqs;
    }
    // 3. swapped requests come back (FIFO) while memory and budget allow
    while (!swapped.empty() && budget_seqs > 0 && budget_tokens > 0) {
      Request* r = swapped.front();
      const int32_t n = tokens_for(r, budget_tokens);
      const int32_t blocks = (int32_t)r->mapping.size() + blocks_needed(r, n);
      if (gpu.num_free() - blocks < watermark_blocks()) break;
      swapped.pop_front();
      for (auto& c : r->mapping) {                    // CPU blocks back to GPU blocks
        int32_t g = -1;
        gpu.alloc(&g);
        swap_in.push_back(c);
        swap_in.push_back(g);
        cpu.release(c);
        c = g;
      }
      set_state(r, kRunning);
      running.push_back(r);
      append_tokens(r, n);
      grants.emplace_back(r, n);
      budget_tokens -= n;
      --budget_seqs;
    }
    // 4. waiting requests are admitted (FCFS) above the watermark; an idle
    //    engine admits its first request whatever the watermark says
    while (!waiting.empty() && swapped.empty() && preempted_ids.empty() && budget_seqs > 0 && budget_tokens > 0) {
      Request* r = waiting.front();
      const int32_t n = tokens_for(r, budget_tokens);
      const int32_t blocks = (n + cfg.block_size - 1) / cfg.block_size;
      const int32_t floor = running.empty() ? 0 : watermark_blocks();
      if (gpu.num_free() - blocks < floor) break;
      waiting.pop_front();
      r->has_table = true;
      r->mapping.clear();
      r->table_tokens = 0;
      append_tokens(r, n);
      set_state(r, kRunning);
      running.push_back(r);
      grants.emplace_back(r, n);
      budget_tokens -= n;
      --budget_seqs;
    }
    // rows: decode rows first, then prefill chunks, each in admission order
    std::stable_sort(grants.begin(), grants.end(), [](const std::pair<Request*, int32_t>& x,
                                                      const std::pair<Request*, int32_t>& y) {
      const bool px = x.first->in_prefill() || x.second > 1, py = y.first->in_prefill() || y.second > 1;
      if (px != py) return !px;
      return x.first->arrival < y.first->arrival;
    });
    int32_t width = 1;
    for (auto& g : grants) width = std::max(width, (int32_t)g.first->mapping.size());
    const size_t B = grants.size();
    tables.assign(B * (size_t)width, -1);
    qsl.push_back(0);
    for (size_t i = 0; i < B; ++i) {
      Request* r = grants[i].first;
      const int32_t n = grants[i].second;
      req_id.push_back(r->id);
      start.push_back(r->num_computed);
      row_tokens.push_back(n);
      is_prefill.push_back(r->in_prefill() || n > 1);
      std::copy(r->mapping.begin(), r->mapping.end(), tables.begin() + i * (size_t)width);
      for (int32_t k = 0; k < n; ++k) positions.push_back(r->num_computed + k);
      qsl.push_back(qsl.back() + n);
      seq_lens.push_back(r->num_computed + n);
    }
    table_width = width;
    pending = true;
  }
  int32_t table_width = 1;
};

namespace {
int bad(const char* msg) { return pkv::report(PKV_EINVAL, msg); }
}  // namespace

extern "C" {

pkv_sched* pkv_sched_create(const pkv_sched_config* c, const int32_t* gpu_order) {
  if (!c) { bad("null config"); return nullptr; }
  if (c->block_size <= 0 || c->num_gpu_blocks <= 0 || c->max_num_seqs <= 0 || c->max_num_batched_tokens <= 0 ||
      c->max_prefill_chunk <= 0 || c->num_cpu_blocks < 0 || !(c->watermark >= 0.0 && c->watermark < 1.0)) {
    bad("sizes must be positive and 0 <= watermark < 1");
    return nullptr;
  }
  if (c->preemption_swap && c->num_cpu_blocks <= 0) {
    bad("swap preemption needs num_cpu_blocks > 0");
    return nullptr;
  }
  if (gpu_order) {
    std::vector<char> seen(c->num_gpu_blocks, 0);
    for (int32_t i = 0; i < c->num_gpu_blocks; ++i) {
      const int32_t b = gpu_order[i];
      if (b < 0 || b >= c->num_gpu_blocks || seen[b]) {
        bad("gpu_order must be a permutation of 0..num_gpu_blocks-1");
        return nullptr;
      }
      seen[b] = 1;
    }
  }
  auto* s = new pkv_sched();
  s->cfg = *c;
  s->gpu.init(c->num_gpu_blocks, gpu_order);
  s->cpu.init(c->num_cpu_blocks, nullptr);
  pkv::report(PKV_OK, "");
  return s;
}

void pkv_sched_destroy(pkv_sched* s) { delete s; }

int pkv_sched_add_request(pkv_sched* s, int64_t req_id, int32_t prompt_len, int32_t max_new_tokens) {
  if (!s) return bad("null scheduler");
  if (s->reqs.count(req_id)) return bad("duplicate request id");
  if (prompt_len <= 0 || max_new_tokens <= 0) return bad("prompt_len and max_new_tokens must be positive");
  const int64_t need = ((int64_t)prompt_len + max_new_tokens + s->cfg.block_size - 1) / s->cfg.block_size;
  if (need > s->cfg.num_gpu_blocks) return bad("request needs more blocks than the pool has");
  auto r = std::make_unique<Request>();
  r->id = req_id;
  r->prompt_len = prompt_len;
  r->max_new = max_new_tokens;
  r->arrival = s->arrivals++;
  s->waiting.push_back(r.get());
  ++s->counts[kWaiting];
  s->reqs.emplace(req_id, std::move(r));
  return pkv::report(PKV_OK, "");
}

int pkv_sched_has_work(const pkv_sched* s) {
  return s && (!s->waiting.empty() || !s->running.empty() || !s->swapped.empty());
}

int pkv_sched_schedule(pkv_sched* s, pkv_sched_plan* p) {
  if (!s || !p) return bad("null pointer");
  if (s->pending) return bad("the previous plan was not completed");
  s->schedule();
  p->num_rows = (int32_t)s->req_id.size();
  p->num_tokens = s->qsl.back();
  p->req_id = s->req_id.data();
  p->start = s->start.data();
  p->row_tokens = s->row_tokens.data();
  p->is_prefill = s->is_prefill.data();
  p->table_width = s->table_width;
  p->block_tables = s->tables.data();
  p->positions = s->positions.data();
  p->query_start_loc = s->qsl.data();
  p->seq_lens = s->seq_lens.data();
  p->num_swap_out = (int32_t)(s->swap_out.size() / 2);
  p->swap_out = s->swap_out.data();
  p->num_swap_in = (int32_t)(s->swap_in.size() / 2);
  p->swap_in = s->swap_in.data();
  p->num_finished = (int32_t)s->finished_ids.size();
  p->finished_ids = s->finished_ids.data();
  p->num_preempted = (int32_t)s->preempted_ids.size();
  p->preempted_ids = s->preempted_ids.data();
  return pkv::report(PKV_OK, "");
}

int pkv_sched_complete(pkv_sched* s) {
  if (!s) return bad("null scheduler");
  if (!s->pending) return bad("no plan to complete");
  for (size_t i = 0; i < s->req_id.size(); ++i) {
    Request* r = s->reqs[s->req_id[i]].get();
    r->num_computed += s->row_tokens[i];
  }
  s->pending = false;
  return pkv::report(PKV_OK, "");
}

int32_t pkv_sched_num_free_gpu(const pkv_sched* s) { return s ? s->gpu.num_free() : 0; }
int32_t pkv_sched_num_free_cpu(const pkv_sched* s) { return s ? s->cpu.num_free() : 0; }
int32_t pkv_sched_count(const pkv_sched* s, int32_t state) {
  return (s && state >= 0 && state < 4) ? s->counts[state] : 0;
}

int pkv_sched_request_info(const pkv_sched* s, int64_t req_id, int32_t* num_computed, int32_t* recompute_to,
                           int32_t* state) {
  if (!s) return bad("null scheduler");
  auto it = s->reqs.find(req_id);
  if (it == s->reqs.end()) return bad("unknown request id");
  if (num_computed) *num_computed = it->second->num_computed;
  if (recompute_to) *recompute_to = it->second->recompute_to;
  if (state) *state = it->second->state;
  return pkv::report(PKV_OK, "");
}

}  // extern "C"

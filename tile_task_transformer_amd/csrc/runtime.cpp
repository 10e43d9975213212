// Tiled tensors, the sequential-task-flow executor, and their C ABI.
#include "runtime.hpp"

#include <algorithm>
#include <queue>
#include <cstdlib>
#include <cstring>
#include <fstream>

namespace tt {

static thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[1024];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}
void clear_error() { g_err.clear(); }

}  // namespace tt

extern "C" const char* tt_last_error(void) { return tt::g_err.c_str(); }
extern "C" const char* tt_version(void) { return "tiletask 0.1 gfx950"; }

using namespace tt;

// ------------------------------------------------------------------ tensors

void tt_tensor::extent(int64_t l, int64_t* ext) const {
  for (int d = 0; d < ndim; ++d) {
    int64_t i = l % grid[d];
    l /= grid[d];
    ext[d] = std::min(tshape[d], shape[d] - i * tshape[d]);
  }
}

int64_t tt_tensor::tile_elems(int64_t l) const {
  int64_t ext[TT_MAX_DIMS];
  extent(l, ext);
  int64_t n = 1;
  for (int d = 0; d < ndim; ++d) n *= ext[d];
  return n;
}

int64_t tt_tensor::lin(const int64_t* idx) const {
  int64_t l = 0;
  for (int d = ndim - 1; d >= 0; --d) l = l * grid[d] + idx[d];
  return l;
}

void tt_tensor::mat(int64_t l, int64_t* rows, int64_t* cols) const {
  int64_t ext[TT_MAX_DIMS];
  extent(l, ext);
  int64_t r = 1, c = 1;
  for (int d = 0; d < ndim; ++d) (d < mat_split ? r : c) *= ext[d];
  *rows = r;
  *cols = c;
}

void* tt_tensor::dev(int64_t l) const {
  if (home == TT_HOME_PINNED_HOST) return res[l].dev;
  if (!base) return nullptr;
  return base + tile_off[l] * (int64_t)esize();
}

namespace tt {

int tensor_create(tt_ctx* ctx, int ndim, const int64_t* shape, const int64_t* tshape, int dtype,
                  int home, int mat_split, const char* name, tt_tensor** out) {
  if (!ctx || !out || !shape || !tshape) return fail(TT_ERR_ARG, "tensor_create: null argument");
  if (ndim < 1 || ndim > TT_MAX_DIMS) return fail(TT_ERR_ARG, "tensor_create: ndim %d out of range", ndim);
  if (dtype != TT_F32 && dtype != TT_I32) return fail(TT_ERR_ARG, "tensor_create: bad dtype");
  if (home != TT_HOME_DEVICE && home != TT_HOME_PINNED_HOST) return fail(TT_ERR_ARG, "tensor_create: bad home");
  std::unique_ptr<tt_tensor> t(new tt_tensor());
  t->ctx = ctx;
  t->id = ctx->next_tensor_id++;
  t->ndim = ndim;
  t->dtype = dtype;
  t->home = home;
  t->mat_split = std::max(0, std::min(mat_split, ndim));
  t->name = name ? name : "";
  t->ntiles = 1;
  t->elems = 1;
  for (int d = 0; d < ndim; ++d) {
    if (shape[d] <= 0 || tshape[d] <= 0)
      return fail(TT_ERR_SHAPE, "tensor %s: axis %d has shape %lld tile %lld", t->name.c_str(), d,
                  (long long)shape[d], (long long)tshape[d]);
    t->shape[d] = shape[d];
    t->tshape[d] = std::min(tshape[d], shape[d]);
    t->grid[d] = ceil_div(shape[d], t->tshape[d]);
    t->ntiles *= t->grid[d];
    t->elems *= shape[d];
  }
  t->tile_off.resize(t->ntiles);
  int64_t off = 0;
  for (int64_t l = 0; l < t->ntiles; ++l) {
    t->tile_off[l] = off;
    off += t->tile_elems(l);
  }
  t->state.resize(t->ntiles);
  if (!ctx->dryrun) {
    if (home == TT_HOME_DEVICE) {
      hipError_t e = hipMalloc(&t->base, std::max<int64_t>(t->bytes(), 256));
      if (e != hipSuccess)
        return fail(TT_ERR_OOM, "tensor %s: hipMalloc(%lld) failed: %s", t->name.c_str(),
                    (long long)t->bytes(), hipGetErrorString(e));
    } else {
      hipError_t e = hipHostMalloc(&t->host, std::max<int64_t>(t->bytes(), 256), hipHostMallocDefault);
      if (e != hipSuccess)
        return fail(TT_ERR_OOM, "tensor %s: hipHostMalloc(%lld) failed: %s", t->name.c_str(),
                    (long long)t->bytes(), hipGetErrorString(e));
      memset(t->host, 0, t->bytes());
      t->res.resize(t->ntiles);
      ctx->has_pinned++;
    }
    t->owned = true;
  }
  ctx->tensors.push_back(t.get());
  *out = t.release();
  return TT_OK;
}

}  // namespace tt

// ----------------------------------------------------------------- executor

tt::Launched* tt_ctx::info(int64_t id) {
  if (id < launched_base || id - launched_base >= (int64_t)launched.size()) return nullptr;
  tt::Launched* li = &launched[id - launched_base];
  // a window's entries are made before its launches; one whose launch
  // stopped on an error leaves entries with no stream
  return li->stream >= 0 ? li : nullptr;
}

int tt_ctx::acquire_event(int* idx) {
  if (events_used == (int)events.size()) {
    hipEvent_t e;
    TT_HIP_TRY(hipEventCreateWithFlags(&e, hipEventDisableTiming));
    events.push_back(e);
  }
  *idx = events_used++;
  stats.events_recorded++;
  return TT_OK;
}

// events that order the executor against streams it does not own: each
// hipStreamWaitEvent takes the event's state at the time of the call, so a
// small fixed set is reused
int tt_ctx::ext_events_init() {
  const size_t want = streams.size() + 3;
  while (ext_events.size() < want) {
    hipEvent_t e;
    TT_HIP_TRY(hipEventCreateWithFlags(&e, hipEventDisableTiming));
    ext_events.push_back(e);
  }
  return TT_OK;
}

int tt_ctx::ensure_workspace(size_t bytes) {
  if (bytes <= workspace_bytes || dryrun) {
    workspace_bytes = std::max(workspace_bytes, bytes);
    return TT_OK;
  }
  int rc = wait_all();
  if (rc) return rc;
  for (void* p : workspace)
    if (p) (void)hipFree(p);
  workspace.assign(n_streams, nullptr);
  ++workspace_gen;
  for (int s = 0; s < n_streams; ++s) {
    hipError_t e = hipMalloc(&workspace[s], bytes);
    if (e != hipSuccess) return fail(TT_ERR_OOM, "workspace hipMalloc(%zu) failed", bytes);
  }
  workspace_bytes = bytes;
  return TT_OK;
}

int tt_ctx::submit(const char* label, std::vector<tt::Access> acc, tt::LaunchFn run, double cost) {
  if (latched) return fail(TT_ERR_STATE, "context has a latched error: %s", latched_msg.c_str());
  auto t0 = std::chrono::steady_clock::now();
  tt::Task task;
  task.id = next_id++;
  snprintf(task.label, sizeof(task.label), "%s", label ? label : "");
  // merge duplicate accesses to the same tile: any write makes it a write
  for (size_t i = 0; i < acc.size(); ++i) {
    if (!acc[i].ref.t) return fail(TT_ERR_ARG, "task %s: null tensor in access %zu", task.label, i);
    if (acc[i].ref.t->ctx != this) return fail(TT_ERR_ARG, "task %s: tensor from another context", task.label);
    if (acc[i].ref.lin < 0 || acc[i].ref.lin >= acc[i].ref.t->ntiles)
      return fail(TT_ERR_ARG, "task %s: tile index out of range", task.label);
  }
  std::vector<tt::Access> merged;
  for (auto& a : acc) {
    bool found = false;
    for (auto& m : merged)
      if (m.ref.t == a.ref.t && m.ref.lin == a.ref.lin) {
        m.mode |= a.mode;
        found = true;
      }
    if (!found) merged.push_back(a);
  }
  // dependency inference (sequential task flow)
  for (auto& a : merged) {
    tt::TileState& st = a.ref.t->state[a.ref.lin];
    if (st.last_writer >= done_below) task.deps.push_back(st.last_writer);
    if (a.mode & TT_W) {
      for (int64_t r : st.readers)
        if (r >= done_below) task.deps.push_back(r);
      st.readers.clear();
      st.last_writer = task.id;
    } else {
      st.readers.push_back(task.id);
    }
  }
  std::sort(task.deps.begin(), task.deps.end());
  task.deps.erase(std::unique(task.deps.begin(), task.deps.end()), task.deps.end());
  stats.tasks++;
  stats.edges += (int64_t)task.deps.size();
  task.acc = std::move(merged);
  task.run = std::move(run);
  task.cost = cost;
  if (pending.empty()) window_base = task.id;
  pending.push_back(std::move(task));
  int rc = TT_OK;
  if ((int)pending.size() >= window) rc = flush();
  stats.submit_seconds += std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
  return rc;
}

// flush_window, with an error that stops a window part way latched (later
// submits and waits report it) and the window dropped, so that none of its
// tasks is launched twice
int tt_ctx::flush() {
  const int rc = flush_window();
  if (rc != TT_OK && !latched) {
    latched = rc;
    latched_msg = std::string("launch: ") + tt_last_error();
  }
  if (rc != TT_OK && !pending.empty()) {
    pending.clear();
    unplan_window();
  }
  return rc;
}

int tt_ctx::flush_window() {
  if (pending.empty()) return latched;
  // 1. stream assignment: continue the chain of a dependency that is still the
  //    tail of its stream, else spread independent work round-robin. With a
  //    heavy lane, tasks of at least heavy_flops run in order on stream 0
  //    (a kernel that fills every CU gains nothing from sharing the GPU with
  //    another such kernel) and the light ones use the other streams, where
  //    they overlap with it.
  const bool lane = heavy_flops > 0 && active_streams > 1;
  const int lo = lane ? 1 : 0;
  for (auto& task : pending) {
    int best = -1;
    if (lane && task.cost >= heavy_flops) {
      best = 0;
    } else {
      int64_t best_id = -1;
      for (int64_t d : task.deps) {
        int ds = -1;
        if (d >= window_base) ds = pending[d - window_base].stream;
        else if (auto* li = info(d)) ds = li->stream;
        if (ds >= lo && ds < active_streams && last_assigned[ds] == d && d > best_id) {
          best = ds;
          best_id = d;
        }
      }
      if (best < 0) {
        best = lo + (rr - lo + (active_streams - lo)) % (active_streams - lo);
        rr = lo + (best - lo + 1) % (active_streams - lo);
      }
    }
    task.stream = best;
    last_assigned[best] = task.id;
  }
  // 2. events only where a successor in this window sits on another stream
  for (auto& task : pending)
    for (int64_t d : task.deps)
      if (d >= window_base && pending[d - window_base].stream != task.stream)
        pending[d - window_base].need_event = true;
  // 3. launch in submission order, or (priorities) in a list-schedule order
  if (launched.empty()) launched_base = window_base;
  if (!dryrun && has_pinned) plan_window();
  const std::vector<size_t> order = launch_order();
  const size_t lbase = launched.size();  // launched[lbase + ti] = pending[ti] (ids are consecutive)
  launched.resize(lbase + pending.size());
  for (size_t oi = 0; oi < order.size(); ++oi) {
    const size_t ti = order[oi];
    tt::Task& task = pending[ti];
    const int s = task.stream;
    cur_task = task.id;
    for (int64_t d : task.deps) {
      if (d < done_below) continue;
      tt::Launched* li = info(d);
      if (!li || li->stream == s) continue;
      if (waited[s][li->stream] >= li->seq) continue;
      if (!dryrun) {
        if (li->event < 0) {
          // dependency launched in an earlier window without an event: record
          // one now on its stream (covers it and whatever followed it there)
          int ev;
          if (int rc = acquire_event(&ev)) return rc;
          TT_HIP_TRY(hipEventRecord(events[ev], streams[li->stream]));
          li->event = ev;
          li->seq = stream_seq[li->stream];
        }
        TT_HIP_TRY(hipStreamWaitEvent(streams[s], events[li->event], 0));
      }
      waited[s][li->stream] = li->seq;
      stats.cross_stream_waits++;
    }
    if (record) {
      tt::TaskRecord r;
      r.id = task.id;
      r.label = task.label;
      r.stream = s;
      r.deps = task.deps;
      r.cost = task.cost;
      for (auto& a : task.acc) r.acc.push_back({a.ref.t->id, {a.ref.lin, a.mode}});
      records.push_back(std::move(r));
    }
    tt::Launched li;
    li.stream = s;
    li.seq = ++stream_seq[s];
    if (!dryrun && !latched) {
      int rc = make_resident(task, streams[s]);
      const bool prof = prof_on && (prof_filter == "*" || prof_filter == task.label) && prof_seen++ % prof_every == 0;
      if (prof && rc == TT_OK) {
        for (int k = 0; k < 2; ++k)
          if (prof_used + k >= (int)prof_events.size()) {
            // timing events only order against this device's own work: no
            // system-scope fence (with it every record drains the caches and
            // stalls the queue a few microseconds)
            hipEvent_t e;
            TT_HIP_TRY(hipEventCreateWithFlags(&e, hipEventDisableSystemFence));
            prof_events.push_back(e);
          }
        prof_pending.push_back({task.label, prof_used, prof_used + 1});
        prof_used += 2;
        TT_HIP_TRY(hipEventRecord(prof_events[prof_pending.back().ev0], streams[s]));
      }
      if (rc == TT_OK && task.run) rc = task.run(streams[s], workspace.empty() ? nullptr : workspace[s]);
      if (prof && rc == TT_OK) TT_HIP_TRY(hipEventRecord(prof_events[prof_pending.back().ev1], streams[s]));
      if (rc != TT_OK) {
        latched = rc;
        latched_msg = std::string(task.label) + ": " + tt_last_error();
      }
      if (task.need_event && !latched) {
        int ev;
        if (int rc2 = acquire_event(&ev)) return rc2;
        TT_HIP_TRY(hipEventRecord(events[ev], streams[s]));
        li.event = ev;
      }
    }
    launched[lbase + ti] = li;
    if (!dryrun && !latched && arena) {
      int rc = clean_ahead(ti);
      if (rc == TT_OK) rc = prefetch(ti);
      if (rc != TT_OK && !latched) {
        latched = rc;
        latched_msg = std::string("prefetch: ") + tt_last_error();
      }
    }
  }
  pending.clear();
  unplan_window();
  if (latched) return fail(latched, "%s", latched_msg.c_str());
  return TT_OK;
}

// Launch order of the pending window. Without priorities (or with
// pinned-host tiles, whose staging plan follows submission order): the
// submission order. With priorities: a list schedule over the window's
// graph -- of the tasks whose dependencies in the window have all been
// launched, the one with the largest bottom level goes next (its cost plus
// the costliest chain of successors to the end of the window; memory-bound
// tasks count as 1 MFLOP, about a microsecond of launch and run time), ties
// by submission order. Every task follows its dependencies, so the order is
// topological; results do not change (the kernels and their per-tile order
// are the same), only which independent task reaches its stream first.
std::vector<size_t> tt_ctx::launch_order() {
  const size_t n = pending.size();
  std::vector<size_t> order(n);
  for (size_t i = 0; i < n; ++i) order[i] = i;
  if (!priorities || has_pinned || n < 2) return order;
  std::vector<std::vector<size_t>> succ(n);
  std::vector<int> indeg(n, 0);
  for (size_t i = 0; i < n; ++i)
    for (int64_t d : pending[i].deps)
      if (d >= window_base) {
        succ[(size_t)(d - window_base)].push_back(i);
        indeg[i]++;
      }
  std::vector<double> bl(n, 0.0);
  for (size_t k = n; k-- > 0;) {
    double m = 0.0;
    for (size_t j : succ[k]) m = std::max(m, bl[j]);
    bl[k] = std::max(pending[k].cost, 1e6) + m;
  }
  auto lower = [&](size_t a, size_t b) { return bl[a] < bl[b] || (bl[a] == bl[b] && a > b); };
  std::priority_queue<size_t, std::vector<size_t>, decltype(lower)> ready(lower);
  for (size_t i = 0; i < n; ++i)
    if (!indeg[i]) ready.push(i);
  size_t k = 0;
  while (!ready.empty()) {
    const size_t i = ready.top();
    ready.pop();
    order[k++] = i;
    for (size_t j : succ[i])
      if (--indeg[j] == 0) ready.push(j);
  }
  return order;
}

// ---------------------------------------------------------------- residency
//
// Tiles whose home is pinned host RAM are staged into a device arena of
// `budget` bytes before a task touches them: H2D copies on the copy stream,
// and a task's stream waits for the copy stream before it runs. When the
// arena is full, the tile whose next use in the launching window is
// farthest is evicted (never one the launching task accesses; tiles
// prefetched for the next tasks last). A tile a task changed is written
// back on a second stream (the host link is full duplex) after every
// launched task that used it; its range is reused, and the tile reloaded,
// only after that write-back. A task writing a tile (TT_W) overwrites all
// of it, so no copy-in is needed for it.

int tt_ctx::arena_init() {
  if (arena) return TT_OK;
  size_t bytes = budget;
  if (!bytes) {
    size_t fr = 0, tot = 0;
    TT_HIP_TRY(hipMemGetInfo(&fr, &tot));
    bytes = fr / 2;
  }
  bytes &= ~(size_t)255;
  hipError_t e = hipMalloc(&arena, bytes);
  if (e != hipSuccess) return fail(TT_ERR_OOM, "residency arena hipMalloc(%zu) failed", bytes);
  arena_bytes = bytes;
  arena_free.clear();
  arena_free[0] = bytes;
  return TT_OK;
}

void tt_ctx::arena_release(size_t off, size_t bytes) {
  auto it = arena_free.emplace(off, bytes).first;
  auto nx = std::next(it);
  if (nx != arena_free.end() && it->first + it->second == nx->first) {
    it->second += nx->second;
    arena_free.erase(nx);
  }
  if (it != arena_free.begin()) {
    auto pv = std::prev(it);
    if (pv->first + pv->second == it->first) {
      pv->second += it->second;
      arena_free.erase(it);
    }
  }
}

// First-fit allocation of `bytes` (rounded to 256) in the arena, evicting
// until a hole fits. Tiles of the task being launched are never evicted;
// tiles prefetched for the next tasks only when nothing else frees room.
// With `soft` (a prefetch for a task with id `use`) the prefetched tiles are
// spared, only tiles needed later than `use` are evicted, and 1 is
// returned, with no error set, when no room can be made.
int tt_ctx::arena_alloc(size_t bytes, size_t* off, bool soft, int64_t use) {
  bytes = (bytes + 255) & ~(size_t)255;
  if (bytes > arena_bytes)
    return fail(TT_ERR_OOM, "tile of %zu bytes exceeds the device budget of %zu bytes", bytes, arena_bytes);
  for (;;) {
    for (auto it = arena_free.begin(); it != arena_free.end(); ++it)
      if (it->second >= bytes) {
        *off = it->first;
        const size_t rest = it->second - bytes, at = it->first + bytes;
        arena_free.erase(it);
        if (rest) arena_free[at] = rest;
        return TT_OK;
      }
    int rc = evict_one(true, soft ? use : -1);
    if (rc == 1 && !soft) rc = evict_one(false, -1);
    if (rc == 1) {
      if (soft) return 1;
      return fail(TT_ERR_OOM, "device budget of %zu bytes cannot hold the tiles one task needs", arena_bytes);
    }
    if (rc) return rc;
  }
}

// `s` waits for every launched task that used the device copy of (t, lin)
int tt_ctx::wait_users(tt_tensor* t, int64_t lin, hipStream_t s) {
  for (int64_t u : t->res[lin].users) {
    if (u < done_below || u >= cur_task) continue;
    tt::Launched* li = info(u);
    if (!li) continue;
    if (li->event < 0) {
      int ev;
      if (int rc = acquire_event(&ev)) return rc;
      TT_HIP_TRY(hipEventRecord(events[ev], streams[li->stream]));
      li->event = ev;
      li->seq = stream_seq[li->stream];
    }
    TT_HIP_TRY(hipStreamWaitEvent(s, events[li->event], 0));
  }
  return TT_OK;
}

// id of the next task in the launching window that accesses the tile
// (INT64_MAX: none)
int64_t tt_ctx::next_use(tt::Residency& r) {
  while (r.fpos < r.future.size() && r.future[r.fpos] < cur_task) ++r.fpos;
  return r.fpos < r.future.size() ? r.future[r.fpos] : INT64_MAX;
}

// `s` must not touch arena range [off, off + bytes) before the write-backs
// that freed any part of it have finished
int tt_ctx::wait_dirty_free(size_t off, size_t bytes, hipStream_t s) {
  for (const DirtyFree& d : dirty_free)
    if (d.off < off + bytes && off < d.off + d.bytes) TT_HIP_TRY(hipStreamWaitEvent(s, events[d.event], 0));
  return TT_OK;
}

// Evict the tile whose next use in the launching window is farthest
// (Belady's rule over the known future; ties: a clean tile, whose eviction
// costs no write-back, then the least recently used). Never a tile of the
// task being launched; with `spare_prefetched`, never one prefetched for an
// upcoming task; with `later_than` >= 0, only a tile next used after that
// task. Returns 1, with no error set, when there is no such tile.
int tt_ctx::evict_one(bool spare_prefetched, int64_t later_than) {
  int best = -1;
  int64_t best_use = -1;
  for (size_t i = 0; i < resident.size(); ++i) {
    tt::Residency& r = resident[i].t->res[resident[i].lin];
    if (r.need >= cur_task) continue;
    if (spare_prefetched && r.protect >= cur_task) continue;
    const int64_t u = next_use(r);
    if (later_than >= 0 && u <= later_than) continue;
    bool better = best < 0 || u > best_use;
    if (!better && u == best_use) {
      const tt::Residency& b = resident[best].t->res[resident[best].lin];
      const bool rc = r.host_valid || !r.dev_valid, bc = b.host_valid || !b.dev_valid;
      better = (rc && !bc) || (rc == bc && r.last_use < b.last_use);
    }
    if (better) {
      best = (int)i;
      best_use = u;
    }
  }
  if (best < 0) return 1;
  tt::TileRef v = resident[best];
  tt::Residency& r = v.t->res[v.lin];
  if (r.dev_valid && !r.host_valid) {
    // write-back on its own stream after every launched user; the range is
    // reused (and the tile reloaded) only after it
    if (int rc = wait_users(v.t, v.lin, d2h_stream)) return rc;
    TT_HIP_TRY(hipMemcpyAsync(v.t->host + v.t->tile_off[v.lin] * 4, r.dev, v.t->tile_elems(v.lin) * 4,
                              hipMemcpyDeviceToHost, d2h_stream));
    int ev;
    if (int rc = acquire_event(&ev)) return rc;
    TT_HIP_TRY(hipEventRecord(events[ev], d2h_stream));
    dirty_free.push_back({r.off, r.bytes, ev});
    r.wb_event = ev;
    stats.d2h_bytes += v.t->tile_elems(v.lin) * 4;
    r.host_valid = true;
  } else {
    // the next writer of the range is an H2D copy, or a task ordered after the
    // copy stream: the copy stream waits for the tile's users, and for an
    // early write-back still reading the range
    if (int rc = wait_users(v.t, v.lin, copy_stream)) return rc;
    if (r.wb_event >= 0) dirty_free.push_back({r.off, r.bytes, r.wb_event});
  }
  arena_release(r.off, r.bytes);
  r.dev = nullptr;
  r.dev_valid = false;
  r.ready_event = -1;
  r.users.clear();
  resident[best] = resident.back();
  resident.pop_back();
  stats.evictions++;
  return TT_OK;
}

// device copy for tile (t, lin), allocated and (if `load`) filled from host;
// `soft`/`use` as for arena_alloc (returns 1 when a prefetch finds no room)
static int stage_tile(tt_ctx* c, tt_tensor* t, int64_t lin, bool load, bool soft, int64_t use) {
  tt::Residency& r = t->res[lin];
  auto mark = [&]() {  // copy-stream work for this tile: it gets the next ready event
    if (!r.staged) {
      r.staged = true;
      c->staged.push_back(&r);
    }
  };
  if (!r.dev) {
    size_t off;
    const size_t bytes = (size_t)t->tile_elems(lin) * 4;
    if (int rc = c->arena_alloc(bytes, &off, soft, use)) return rc;
    r.dev = (float*)(c->arena + off);
    r.off = off;
    r.bytes = (bytes + 255) & ~(size_t)255;
    r.dev_valid = false;
    c->resident.push_back(tt::TileRef{t, lin});
    // whoever writes the range next (this copy, or the task through the
    // tile's ready event on the copy stream) comes after the write-backs
    // that freed it, and after the users of evicted occupants (the copy
    // stream waited for them when they were evicted)
    if (int rc = c->wait_dirty_free(r.off, r.bytes, c->copy_stream)) return rc;
    mark();
  }
  if (load && !r.dev_valid) {
    if (!r.host_valid) return fail(TT_ERR_STATE, "tile has neither a valid host nor device copy");
    if (r.wb_event >= 0) TT_HIP_TRY(hipStreamWaitEvent(c->copy_stream, c->events[r.wb_event], 0));
    TT_HIP_TRY(hipMemcpyAsync(r.dev, t->host + t->tile_off[lin] * 4, t->tile_elems(lin) * 4, hipMemcpyHostToDevice,
                              c->copy_stream));
    c->stats.h2d_bytes += t->tile_elems(lin) * 4;
    r.dev_valid = true;
    mark();
  }
  return TT_OK;
}

// one event on the copy stream after everything staged since the last one
int tt_ctx::mark_ready() {
  if (staged.empty()) return TT_OK;
  int ev;
  if (int rc = acquire_event(&ev)) return rc;
  TT_HIP_TRY(hipEventRecord(events[ev], copy_stream));
  if ((int)ready_seq.size() <= ev) ready_seq.resize(ev + 1, 0);
  ready_seq[ev] = ++ready_count;
  for (tt::Residency* r : staged) {
    r->ready_event = ev;
    r->staged = false;
  }
  staged.clear();
  return TT_OK;
}

int tt_ctx::make_resident(tt::Task& task, hipStream_t s) {
  bool any = false;
  for (auto& a : task.acc)
    if (a.ref.t->home == TT_HOME_PINNED_HOST) {
      if (capturing) return fail(TT_ERR_UNSUPPORTED, "pinned-host tiles cannot be captured into a graph");
      any = true;
      a.ref.t->res[a.ref.lin].need = task.id;
    }
  if (!any) return TT_OK;
  if (int rc = arena_init()) return rc;
  for (auto& a : task.acc) {
    tt_tensor* t = a.ref.t;
    if (t->home != TT_HOME_PINNED_HOST) continue;
    if (int rc = stage_tile(this, t, a.ref.lin, (a.mode & TT_R) != 0, false, task.id)) return rc;
  }
  // the task's stream runs after the copy-stream point at which the last of
  // its tiles became ready (copy-stream events complete in order)
  if (int rc = mark_ready()) return rc;
  int need = -1;
  for (auto& a : task.acc)
    if (a.ref.t->home == TT_HOME_PINNED_HOST) {
      const int ev = a.ref.t->res[a.ref.lin].ready_event;
      if (ev >= 0 && (need < 0 || ready_seq[ev] > ready_seq[need])) need = ev;
    }
  if (need >= 0) {
    const int si = (int)(std::find(streams.begin(), streams.end(), s) - streams.begin());
    if (si < n_streams && waited_copy[si] < ready_seq[need]) {
      TT_HIP_TRY(hipStreamWaitEvent(s, events[need], 0));
      waited_copy[si] = ready_seq[need];
    }
  }
  for (auto& a : task.acc) {
    tt_tensor* t = a.ref.t;
    if (t->home != TT_HOME_PINNED_HOST) continue;
    tt::Residency& r = t->res[a.ref.lin];
    // a write-back of this device copy may still be reading it
    if ((a.mode & TT_W) && r.wb_event >= 0) TT_HIP_TRY(hipStreamWaitEvent(s, events[r.wb_event], 0));
    if (a.mode & TT_W) {
      r.dev_valid = true;
      r.host_valid = false;
      r.users.clear();
    }
    r.users.push_back(task.id);
    r.last_use = task.id;
  }
  return TT_OK;
}

// Record, for every pinned tile the window's tasks access, the ids of those
// tasks: the eviction rule looks them up.
void tt_ctx::plan_window() {
  for (auto& task : pending)
    for (auto& a : task.acc)
      if (a.ref.t->home == TT_HOME_PINNED_HOST) {
        tt::Residency& r = a.ref.t->res[a.ref.lin];
        if (r.future.empty()) planned.push_back(&r);
        if (r.future.empty() || r.future.back() != task.id) r.future.push_back(task.id);
      }
}

void tt_ctx::unplan_window() {
  for (tt::Residency* r : planned) {
    r->future.clear();
    r->fpos = 0;
  }
  planned.clear();
}

// A tile the launched task i wrote that no later task of the window
// accesses is written back now, on the write-back stream after task i: it
// stays resident but clean, so its eviction later copies nothing. A later
// writer of the tile waits for this copy (make_resident), and so does any
// reuse of its range (evict_one).
int tt_ctx::clean_ahead(size_t i) {
  const tt::Task& task = pending[i];
  cur_task = task.id + 1;
  for (auto& a : task.acc) {
    tt_tensor* t = a.ref.t;
    if (t->home != TT_HOME_PINNED_HOST || !(a.mode & TT_W)) continue;
    tt::Residency& r = t->res[a.ref.lin];
    if (!r.dev || !r.dev_valid || r.host_valid || next_use(r) != INT64_MAX) continue;
    if (int rc = wait_users(t, a.ref.lin, d2h_stream)) return rc;
    TT_HIP_TRY(hipMemcpyAsync(t->host + t->tile_off[a.ref.lin] * 4, r.dev, t->tile_elems(a.ref.lin) * 4,
                              hipMemcpyDeviceToHost, d2h_stream));
    int ev;
    if (int rc = acquire_event(&ev)) return rc;
    TT_HIP_TRY(hipEventRecord(events[ev], d2h_stream));
    r.wb_event = ev;
    r.host_valid = true;
    stats.d2h_bytes += t->tile_elems(a.ref.lin) * 4;
  }
  return TT_OK;
}

// Stage the pinned tiles that the next tasks read (up to 16 tasks and a
// quarter of the arena ahead) so their copies overlap the current task; a
// tile written by an earlier one of those tasks is not prefetched (its host
// copy would be stale).
int tt_ctx::prefetch(size_t i) {
  constexpr size_t kAhead = 16;
  const size_t end = std::min(pending.size(), i + 1 + kAhead);
  // task i has been launched: an eviction from here on must wait for it too
  cur_task = pending[i].id + 1;
  size_t planned_bytes = 0;
  for (size_t j = i + 1; j < end; ++j) {
    for (auto& a : pending[j].acc)
      if (a.ref.t->home == TT_HOME_PINNED_HOST) {
        tt::Residency& r = a.ref.t->res[a.ref.lin];
        r.protect = std::max(r.protect, pending[j].id);
      }
    for (auto& a : pending[j].acc) {
      tt_tensor* t = a.ref.t;
      if (t->home != TT_HOME_PINNED_HOST || !(a.mode & TT_R)) continue;
      tt::Residency& r = t->res[a.ref.lin];
      if (r.dev_valid) continue;
      bool written_before = false;
      for (size_t k = i + 1; k < j && !written_before; ++k)
        for (auto& b : pending[k].acc)
          if (b.ref.t == t && b.ref.lin == a.ref.lin && (b.mode & TT_W)) written_before = true;
      if (written_before) continue;
      planned_bytes += (size_t)t->tile_elems(a.ref.lin) * 4;
      if (planned_bytes > arena_bytes / 4) return TT_OK;
      const int rc = stage_tile(this, t, a.ref.lin, true, true, pending[j].id);
      if (rc == 1) return mark_ready();  // no room without evicting what is needed sooner: stop here
      if (rc) return rc;
      stats.prefetches++;
    }
    // task j's tiles get their own ready event: task j + 1 does not wait for
    // the copies of the tasks after it
    if (int rc = mark_ready()) return rc;
  }
  return TT_OK;
}

void tt_ctx::drop_resident(tt_tensor* t) {
  for (size_t i = 0; i < resident.size();)
    if (resident[i].t == t) {
      tt::Residency& r = t->res[resident[i].lin];
      arena_release(r.off, r.bytes);
      r.dev = nullptr;
      resident[i] = resident.back();
      resident.pop_back();
    } else {
      ++i;
    }
}

int tt_ctx::wait_all() {
  if (capturing) return fail(TT_ERR_STATE, "cannot wait while a graph is being captured");
  int rc = flush();
  if (!dryrun) {
    std::vector<hipStream_t> all(streams);
    if (copy_stream) all.push_back(copy_stream);
    if (d2h_stream) all.push_back(d2h_stream);
    for (auto s : all) {
      hipError_t e = hipStreamSynchronize(s);
      if (e != hipSuccess && !latched) {
        latched = TT_ERR_HIP;
        latched_msg = std::string("asynchronous fault: ") + hipGetErrorString(e);
      }
    }
  }
  if (!latched && !dryrun) prof_collect();
  forget_launched();  // everything submitted so far has completed
  if (latched) return fail(latched, "%s", latched_msg.c_str());
  return rc;
}

void tt_ctx::forget_launched() {
  // write-back events are recycled with the others; every reader recorded
  // so far has completed, so no later task needs an edge to it (tiles that
  // are only read, such as parameters in steps without an update, would
  // otherwise collect reader ids without bound)
  for (auto& t : tensors) {
    for (auto& r : t->res) {
      r.wb_event = -1;
      r.ready_event = -1;  // every copy has completed; the event is recycled
    }
    for (auto& st : t->state) st.readers.clear();
  }
  dirty_free.clear();
  done_below = next_id;
  launched.clear();
  launched_base = next_id;
  events_used = 0;
  ready_count = 0;
  for (tt::Residency* r : staged) r->staged = false;  // (only after a failed staging)
  staged.clear();
  std::fill(waited_copy.begin(), waited_copy.end(), 0);
  for (auto& w : waited) std::fill(w.begin(), w.end(), 0);
  for (int s = 0; s < n_streams; ++s) {
    stream_seq[s] = 0;
    last_assigned[s] = -1;
  }
}

// ------------------------------------------------------------ graph capture
//
// Stream 0 starts the capture; every other stream joins it by waiting on an
// event recorded there, so the kernels, copies and event waits the flushes
// issue on any stream become nodes and edges of one graph. At the end every
// stream's tail is joined back into stream 0. Per-task timing and
// pinned-host tiles (whose copies are decided at launch time) are not
// capturable.

int tt_ctx::capture_begin() {
  if (dryrun) return fail(TT_ERR_UNSUPPORTED, "graph capture needs a device context");
  if (capturing) return fail(TT_ERR_STATE, "a capture is already open");
  if (prof_on) return fail(TT_ERR_STATE, "per-task timing is on: it cannot be captured");
  if (int rc = wait_all()) return rc;
  TT_HIP_TRY(hipStreamBeginCapture(streams[0], hipStreamCaptureModeThreadLocal));
  capturing = true;
  int ev;
  if (int rc = acquire_event(&ev)) return rc;
  TT_HIP_TRY(hipEventRecord(events[ev], streams[0]));
  for (int s = 1; s < n_streams; ++s) TT_HIP_TRY(hipStreamWaitEvent(streams[s], events[ev], 0));
  return TT_OK;
}

int tt_ctx::capture_end(hipGraphExec_t* out) {
  if (!capturing) return fail(TT_ERR_STATE, "no capture is open");
  int rc = flush();
  hipError_t e = hipSuccess;
  for (int s = 1; s < n_streams && e == hipSuccess; ++s) {
    int ev;
    if (acquire_event(&ev)) break;
    e = hipEventRecord(events[ev], streams[s]);
    if (e == hipSuccess) e = hipStreamWaitEvent(streams[0], events[ev], 0);
  }
  hipGraph_t graph = nullptr;
  const hipError_t e2 = hipStreamEndCapture(streams[0], &graph);
  capturing = false;
  forget_launched();  // the graph carries the order of what was captured
  if (rc == TT_OK && latched) rc = fail(latched, "%s", latched_msg.c_str());
  if (rc == TT_OK && e != hipSuccess) rc = fail(TT_ERR_HIP, "capture join: %s", hipGetErrorString(e));
  if (rc == TT_OK && e2 != hipSuccess) rc = fail(TT_ERR_HIP, "hipStreamEndCapture: %s", hipGetErrorString(e2));
  if (rc == TT_OK && out) {
    const hipError_t e3 = hipGraphInstantiate(out, graph, nullptr, nullptr, 0);
    if (e3 != hipSuccess) rc = fail(TT_ERR_HIP, "hipGraphInstantiate: %s", hipGetErrorString(e3));
  }
  if (graph) (void)hipGraphDestroy(graph);
  return rc;
}

int tt_ctx::graph_launch(hipGraphExec_t exec) {
  if (latched) return fail(TT_ERR_STATE, "context has a latched error: %s", latched_msg.c_str());
  if (capturing) return fail(TT_ERR_STATE, "cannot launch a graph while capturing");
  if (int rc = flush()) return rc;
  TT_HIP_TRY(hipGraphLaunch(exec, streams[0]));
  // work submitted later, on any stream, runs after the graph
  int ev;
  if (int rc = acquire_event(&ev)) return rc;
  TT_HIP_TRY(hipEventRecord(events[ev], streams[0]));
  for (int s = 1; s < n_streams; ++s) TT_HIP_TRY(hipStreamWaitEvent(streams[s], events[ev], 0));
  forget_launched();
  events_used = ev + 1;  // keep the join event alive until the next drain
  return TT_OK;
}

int tt_ctx::prof_collect() {
  for (auto& r : prof_pending) {
    float ms = 0.f;
    TT_HIP_TRY(hipEventElapsedTime(&ms, prof_events[r.ev0], prof_events[r.ev1]));
    if (prof_base_set) {
      float t0 = 0.f;
      TT_HIP_TRY(hipEventElapsedTime(&t0, prof_base, prof_events[r.ev0]));
      prof_iv.push_back({t0, t0 + ms});
    }
    ProfAgg* a = nullptr;
    for (auto& p : prof_agg)
      if (p.first == r.label) a = &p.second;
    if (!a) {
      prof_agg.push_back({r.label, ProfAgg{}});
      a = &prof_agg.back().second;
    }
    a->count++;
    a->total += ms;
    a->mn = std::min(a->mn, (double)ms);
    a->mx = std::max(a->mx, (double)ms);
  }
  prof_pending.clear();
  prof_used = 0;
  return TT_OK;
}

// -------------------------------------------------------------------- C ABI

namespace {

// tt_ctx_create with the executor's streams either created here or borrowed
// from the caller (not null, pairwise distinct, not destroyed here)
int ctx_create(int device, int n_streams, void* const* borrowed, int window, size_t device_budget_bytes,
               tt_ctx** out) {
  clear_error();
  if (!out) return fail(TT_ERR_ARG, "tt_ctx_create: out is null");
  if (n_streams < 1 || n_streams > 16) return fail(TT_ERR_ARG, "tt_ctx_create: n_streams must be 1..16");
  if (window < 0) return fail(TT_ERR_ARG, "tt_ctx_create: negative window");
  std::unique_ptr<tt_ctx> c(new tt_ctx());
  c->dryrun = device == TT_DEVICE_DRYRUN;
  c->device = c->dryrun ? -1 : device;
  c->n_streams = n_streams;
  c->active_streams = n_streams;
  c->window = window ? window : 512;
  c->budget = device_budget_bytes;
  c->record = c->dryrun;
  if (const char* e = getenv("TT_RECORD_DAG")) c->record = c->record || atoi(e) != 0;
  c->stream_seq.assign(n_streams, 0);
  c->last_assigned.assign(n_streams, -1);
  c->waited.assign(n_streams, std::vector<int64_t>(n_streams, 0));
  c->waited_copy.assign(n_streams, 0);
  if (!c->dryrun) {
    if (device < 0) return fail(TT_ERR_ARG, "tt_ctx_create: bad device %d", device);
    TT_HIP_TRY(hipSetDevice(device));
    c->streams.resize(n_streams);
    for (int s = 0; s < n_streams; ++s) {
      if (borrowed) {
        c->streams[s] = static_cast<hipStream_t>(borrowed[s]);
        continue;
      }
      if (hipError_t e = hipStreamCreateWithFlags(&c->streams[s], hipStreamNonBlocking)) {
        for (int q = 0; q < s; ++q) (void)hipStreamDestroy(c->streams[q]);
        return fail(TT_ERR_HIP, "tt_ctx_create: hipStreamCreateWithFlags: %s", hipGetErrorString(e));
      }
    }
    c->owns_streams = !borrowed;
    hipError_t e = hipStreamCreateWithFlags(&c->copy_stream, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipStreamCreateWithFlags(&c->d2h_stream, hipStreamNonBlocking);
    if (e != hipSuccess) {
      if (c->owns_streams)
        for (auto st : c->streams) (void)hipStreamDestroy(st);
      if (c->copy_stream) (void)hipStreamDestroy(c->copy_stream);
      return fail(TT_ERR_HIP, "tt_ctx_create: hipStreamCreateWithFlags: %s", hipGetErrorString(e));
    }
  }
  *out = c.release();
  return TT_OK;
}

}  // namespace

extern "C" {

int tt_ctx_create(int device, int n_streams, int window, size_t device_budget_bytes, tt_ctx** out) {
  return ctx_create(device, n_streams, nullptr, window, device_budget_bytes, out);
}

int tt_ctx_create_on_streams(int device, int n_streams, void* const* streams, int window,
                             size_t device_budget_bytes, tt_ctx** out) {
  clear_error();
  if (device == TT_DEVICE_DRYRUN) return fail(TT_ERR_ARG, "tt_ctx_create_on_streams: needs a device");
  if (!streams) return fail(TT_ERR_ARG, "tt_ctx_create_on_streams: null stream array");
  if (n_streams < 1 || n_streams > 16) return fail(TT_ERR_ARG, "tt_ctx_create: n_streams must be 1..16");
  for (int i = 0; i < n_streams; ++i) {
    if (!streams[i])
      return fail(TT_ERR_ARG, "tt_ctx_create_on_streams: stream %d is the null (legacy default) stream", i);
    for (int j = 0; j < i; ++j)
      if (streams[j] == streams[i]) return fail(TT_ERR_ARG, "tt_ctx_create_on_streams: streams %d and %d are one stream", j, i);
  }
  return ctx_create(device, n_streams, streams, window, device_budget_bytes, out);
}

int tt_ctx_destroy(tt_ctx* c) {
  clear_error();
  if (!c) return fail(TT_ERR_ARG, "tt_ctx_destroy: null");
  int rc = c->dryrun ? TT_OK : c->wait_all();
  while (!c->tensors.empty()) tt_tensor_destroy(c->tensors.back());
  if (!c->dryrun) {
    for (void* p : c->workspace)
      if (p) (void)hipFree(p);
    for (auto e : c->events) (void)hipEventDestroy(e);
    for (auto e : c->prof_events) (void)hipEventDestroy(e);
    if (c->prof_base) (void)hipEventDestroy(c->prof_base);
    for (auto e : c->ext_events) (void)hipEventDestroy(e);
    if (c->owns_streams)
      for (auto s : c->streams) (void)hipStreamDestroy(s);
    if (c->copy_stream) (void)hipStreamDestroy(c->copy_stream);
    if (c->d2h_stream) (void)hipStreamDestroy(c->d2h_stream);
    if (c->arena) (void)hipFree(c->arena);
  }
  delete c;
  return rc;
}

int tt_ctx_stream(tt_ctx* c, int i, void** stream) {
  if (!c || !stream || i < 0 || i >= c->n_streams) return fail(TT_ERR_ARG, "tt_ctx_stream: bad argument");
  *stream = c->dryrun ? nullptr : (void*)c->streams[i];
  return TT_OK;
}

int tt_ctx_streams_active(tt_ctx* c, int n) {
  if (!c || n < 1 || n > c->n_streams) return fail(TT_ERR_ARG, "tt_ctx_streams_active: n must be 1..n_streams");
  if (int rc = c->flush()) return rc;
  c->active_streams = n;
  return TT_OK;
}

int tt_ctx_heavy_lane(tt_ctx* c, double min_flops) {
  if (!c || !(min_flops >= 0)) return fail(TT_ERR_ARG, "tt_ctx_heavy_lane: bad argument");
  if (int rc = c->flush()) return rc;
  c->heavy_flops = min_flops;
  return TT_OK;
}

int tt_ctx_priorities(tt_ctx* c, int on) {
  if (!c) return fail(TT_ERR_ARG, "tt_ctx_priorities: null");
  if (int rc = c->flush()) return rc;
  c->priorities = on != 0;
  return TT_OK;
}

int tt_ctx_record(tt_ctx* c, int on) {
  if (!c) return fail(TT_ERR_ARG, "tt_ctx_record: null");
  c->record = on != 0;
  return TT_OK;
}

int tt_ctx_profile(tt_ctx* c, const char* label_filter) {
  if (!c) return fail(TT_ERR_ARG, "tt_ctx_profile: null");
  if (c->capturing) return fail(TT_ERR_STATE, "tt_ctx_profile: a graph is being captured");
  // drain first: the reference event below then precedes every timed task
  // on every stream
  if (int rc = c->wait_all()) return rc;
  c->prof_on = label_filter != nullptr;
  c->prof_filter = label_filter ? label_filter : "";
  c->prof_seen = 0;
  c->prof_iv.clear();
  c->prof_base_set = false;
  if (c->prof_on && !c->dryrun) {
    if (!c->prof_base) TT_HIP_TRY(hipEventCreateWithFlags(&c->prof_base, hipEventDisableSystemFence));
    TT_HIP_TRY(hipEventRecord(c->prof_base, c->streams[0]));
    c->prof_base_set = true;
  }
  return TT_OK;
}

int tt_profile_busy(tt_ctx* c, double* busy_ms, double* span_ms, int64_t* n_tasks) {
  clear_error();
  if (!c || !busy_ms || !span_ms || !n_tasks) return fail(TT_ERR_ARG, "tt_profile_busy: bad argument");
  if (int rc = c->wait_all()) return rc;
  auto& iv = c->prof_iv;
  std::sort(iv.begin(), iv.end());
  double busy = 0, lo = 0, hi = 0, first = 0, last = 0;
  for (size_t i = 0; i < iv.size(); ++i) {
    const double a = iv[i].first, b = std::max(iv[i].first, iv[i].second);
    if (i == 0) {
      lo = first = a;
      hi = last = b;
      continue;
    }
    last = std::max(last, b);
    if (a > hi) {
      busy += hi - lo;
      lo = a;
      hi = b;
    } else {
      hi = std::max(hi, b);
    }
  }
  if (!iv.empty()) busy += hi - lo;
  *busy_ms = busy;
  *span_ms = iv.empty() ? 0.0 : last - first;
  *n_tasks = (int64_t)iv.size();
  iv.clear();
  return TT_OK;
}

int tt_ctx_profile_every(tt_ctx* c, int every) {
  if (!c || every < 1) return fail(TT_ERR_ARG, "tt_ctx_profile_every: bad argument");
  c->prof_every = every;
  return TT_OK;
}

int tt_profile_read(tt_ctx* c, tt_profile_entry* out, int max_entries, int* n_entries) {
  clear_error();
  if (!c || !n_entries || (max_entries > 0 && !out)) return fail(TT_ERR_ARG, "tt_profile_read: bad argument");
  if (int rc = c->wait_all()) return rc;
  int n = 0;
  for (auto& p : c->prof_agg) {
    if (n < max_entries) {
      tt_profile_entry& e = out[n];
      memset(&e, 0, sizeof(e));
      snprintf(e.label, sizeof(e.label), "%s", p.first.c_str());
      e.count = p.second.count;
      e.total_ms = p.second.total;
      e.min_ms = p.second.count ? p.second.mn : 0;
      e.max_ms = p.second.mx;
    }
    ++n;
  }
  *n_entries = n;
  c->prof_agg.clear();
  return TT_OK;
}

int tt_tensor_create(tt_ctx* ctx, int ndim, const int64_t* shape, const int64_t* tile_shape, int dtype,
                     int home, tt_tensor** out) {
  clear_error();
  return tt::tensor_create(ctx, ndim, shape, tile_shape, dtype, home, ndim - 1, nullptr, out);
}

int tt_tensor_wrap(tt_ctx* ctx, int ndim, const int64_t* shape, const int64_t* tile_shape, int dtype,
                   void* device_base, tt_tensor** out) {
  clear_error();
  if (!ctx || ctx->dryrun) return fail(TT_ERR_ARG, "tt_tensor_wrap: needs a device context");
  if (!device_base) return fail(TT_ERR_ARG, "tt_tensor_wrap: null base");
  // create a dry descriptor then attach the caller's memory
  bool dr = ctx->dryrun;
  ctx->dryrun = true;
  int rc = tt::tensor_create(ctx, ndim, shape, tile_shape, dtype, TT_HOME_DEVICE, ndim - 1, nullptr, out);
  ctx->dryrun = dr;
  if (rc) return rc;
  (*out)->base = (char*)device_base;
  (*out)->owned = false;
  return TT_OK;
}

int tt_tensor_destroy(tt_tensor* t) {
  if (!t) return fail(TT_ERR_ARG, "tt_tensor_destroy: null");
  tt_ctx* c = t->ctx;
  if (!c->dryrun) {
    int rc = c->wait_all();
    (void)rc;
  }
  c->drop_resident(t);  // device copies live in the context's arena
  if (!t->res.empty()) c->has_pinned--;
  if (t->owned) {
    if (t->base) (void)hipFree(t->base);
    if (t->host) (void)hipHostFree(t->host);
  }
  auto it = std::find(c->tensors.begin(), c->tensors.end(), t);
  if (it != c->tensors.end()) c->tensors.erase(it);
  delete t;
  return TT_OK;
}

int tt_tensor_set_matrix_split(tt_tensor* t, int k) {
  clear_error();
  if (!t || k < 0 || k > t->ndim) return fail(TT_ERR_ARG, "tt_tensor_set_matrix_split: bad argument");
  t->mat_split = k;
  return TT_OK;
}

int64_t tt_tensor_bytes(const tt_tensor* t) { return t ? t->bytes() : -1; }

int tt_tensor_grid(const tt_tensor* t, int64_t* grid_out, int64_t* ntiles) {
  if (!t) return fail(TT_ERR_ARG, "tt_tensor_grid: null");
  if (grid_out)
    for (int d = 0; d < t->ndim; ++d) grid_out[d] = t->grid[d];
  if (ntiles) *ntiles = t->ntiles;
  return TT_OK;
}

static int check_idx(const tt_tensor* t, const int64_t* idx) {
  if (!idx) return fail(TT_ERR_ARG, "null tile index");
  for (int d = 0; d < t->ndim; ++d)
    if (idx[d] < 0 || idx[d] >= t->grid[d])
      return fail(TT_ERR_ARG, "tile index %lld out of range on axis %d", (long long)idx[d], d);
  return TT_OK;
}

int tt_tensor_tile(tt_tensor* t, const int64_t* idx, void** dev_ptr, int64_t* extent) {
  clear_error();
  if (!t) return fail(TT_ERR_ARG, "tt_tensor_tile: null");
  if (int rc = check_idx(t, idx)) return rc;
  int64_t l = t->lin(idx);
  if (!t->ctx->dryrun)
    if (int rc = t->ctx->wait_all()) return rc;
  if (t->home == TT_HOME_PINNED_HOST)
    return fail(TT_ERR_UNSUPPORTED, "tt_tensor_tile: pinned-host tile access not supported");
  if (dev_ptr) *dev_ptr = t->dev(l);
  if (extent) t->extent(l, extent);
  return TT_OK;
}

// dense row-major <-> tile-major permutation on the host
static void permute(const tt_tensor* t, const char* src, char* dst, bool to_tiles) {
  const size_t es = t->esize();
  int64_t dstride[TT_MAX_DIMS];
  dstride[t->ndim - 1] = 1;
  for (int d = t->ndim - 2; d >= 0; --d) dstride[d] = dstride[d + 1] * t->shape[d + 1];
  for (int64_t l = 0; l < t->ntiles; ++l) {
    int64_t ext[TT_MAX_DIMS], org[TT_MAX_DIMS];
    t->extent(l, ext);
    int64_t rem = l;
    for (int d = 0; d < t->ndim; ++d) {
      org[d] = (rem % t->grid[d]) * t->tshape[d];
      rem /= t->grid[d];
    }
    int64_t tile_base = t->tile_off[l];
    const int last = t->ndim - 1;
    int64_t nrows = 1;
    for (int d = 0; d < last; ++d) nrows *= ext[d];
    int64_t cnt[TT_MAX_DIMS] = {};
    for (int64_t r = 0; r < nrows; ++r) {
      int64_t doff = org[last];
      for (int d = 0; d < last; ++d) doff += (org[d] + cnt[d]) * dstride[d];
      int64_t toff = tile_base + r * ext[last];
      if (to_tiles) memcpy(dst + toff * es, src + doff * es, ext[last] * es);
      else memcpy(dst + doff * es, src + toff * es, ext[last] * es);
      for (int d = last - 1; d >= 0; --d) {
        if (++cnt[d] < ext[d]) break;
        cnt[d] = 0;
      }
    }
  }
}

int tt_tensor_copy_in(tt_tensor* t, const void* dense) {
  clear_error();
  if (!t || !dense) return fail(TT_ERR_ARG, "tt_tensor_copy_in: null");
  tt_ctx* c = t->ctx;
  if (c->dryrun) return fail(TT_ERR_STATE, "tt_tensor_copy_in: dry-run context");
  if (int rc = c->wait_all()) return rc;
  std::vector<char> buf(t->bytes());
  permute(t, (const char*)dense, buf.data(), true);
  if (t->home == TT_HOME_PINNED_HOST) {
    memcpy(t->host, buf.data(), t->bytes());
    for (auto& r : t->res) {
      r.host_valid = true;
      r.dev_valid = false;
    }
    return TT_OK;
  }
  TT_HIP_TRY(hipMemcpy(t->base, buf.data(), t->bytes(), hipMemcpyHostToDevice));
  return TT_OK;
}

int tt_tensor_copy_out(tt_tensor* t, void* dense) {
  clear_error();
  if (!t || !dense) return fail(TT_ERR_ARG, "tt_tensor_copy_out: null");
  tt_ctx* c = t->ctx;
  if (c->dryrun) return fail(TT_ERR_STATE, "tt_tensor_copy_out: dry-run context");
  if (int rc = c->wait_all()) return rc;
  std::vector<char> buf(t->bytes());
  if (t->home == TT_HOME_PINNED_HOST) {
    for (int64_t l = 0; l < t->ntiles; ++l) {
      auto& r = t->res[l];
      if (!r.host_valid && r.dev_valid)
        TT_HIP_TRY(hipMemcpy(t->host + t->tile_off[l] * 4, r.dev, t->tile_elems(l) * 4, hipMemcpyDeviceToHost));
      r.host_valid = true;
    }
    memcpy(buf.data(), t->host, t->bytes());
  } else {
    TT_HIP_TRY(hipMemcpy(buf.data(), t->base, t->bytes(), hipMemcpyDeviceToHost));
  }
  permute(t, buf.data(), (char*)dense, false);
  return TT_OK;
}

int tt_submit_nop(tt_ctx* c, const char* label, const tt_access* acc, int n) {
  clear_error();
  if (!c || (n > 0 && !acc) || n < 0) return fail(TT_ERR_ARG, "tt_submit_nop: bad argument");
  std::vector<tt::Access> a;
  for (int i = 0; i < n; ++i) {
    if (!acc[i].tensor) return fail(TT_ERR_ARG, "tt_submit_nop: null tensor");
    if (acc[i].mode < TT_R || acc[i].mode > TT_RW) return fail(TT_ERR_ARG, "tt_submit_nop: bad mode");
    if (int rc = check_idx(acc[i].tensor, acc[i].tile)) return rc;
    a.push_back(tt::Access{tt::TileRef{acc[i].tensor, acc[i].tensor->lin(acc[i].tile)}, acc[i].mode});
  }
  return c->submit(label, std::move(a), nullptr);
}

int tt_submit_gemm(tt_ctx* c, int transA, int transB, float alpha, tt_tensor* A, const int64_t* ia,
                   tt_tensor* B, const int64_t* ib, float beta, tt_tensor* C, const int64_t* ic) {
  clear_error();
  if (!c || !A || !B || !C) return fail(TT_ERR_ARG, "tt_submit_gemm: null");
  if (A->ndim != 2 || B->ndim != 2 || C->ndim != 2) return fail(TT_ERR_SHAPE, "tt_submit_gemm: 2-D tensors only");
  if (A->dtype != TT_F32 || B->dtype != TT_F32 || C->dtype != TT_F32)
    return fail(TT_ERR_ARG, "tt_submit_gemm: f32 tensors only");
  for (auto p : {std::make_pair((const tt_tensor*)A, ia), std::make_pair((const tt_tensor*)B, ib),
                  std::make_pair((const tt_tensor*)C, ic)})
    if (int rc = check_idx(p.first, p.second)) return rc;
  int64_t la = A->lin(ia), lb = B->lin(ib), lc = C->lin(ic);
  int64_t ar, ac, br, bc, cr, cc;
  A->mat(la, &ar, &ac);
  B->mat(lb, &br, &bc);
  C->mat(lc, &cr, &cc);
  int64_t m = transA ? ac : ar, k = transA ? ar : ac;
  int64_t kb = transB ? bc : br, n = transB ? br : bc;
  if (k != kb || m != cr || n != cc)
    return fail(TT_ERR_SHAPE, "tt_submit_gemm: op(A) %lldx%lld, op(B) %lldx%lld, C %lldx%lld", (long long)m,
                (long long)k, (long long)kb, (long long)n, (long long)cr, (long long)cc);
  std::vector<tt::Access> acc = {tt::R(A, la), tt::R(B, lb), beta == 0.f ? tt::W(C, lc) : tt::RW(C, lc)};
  return c->submit("gemm", std::move(acc), [=](hipStream_t s, void*) {
    return tile_gemm(s, transA, transB, m, n, k, alpha, (const float*)A->dev(la), ac, (const float*)B->dev(lb), bc,
                     beta, (float*)C->dev(lc), cc, TT_EPI_NONE, nullptr, nullptr, 0, nullptr, 0);
  }, 2.0 * m * n * k);
}

int tt_submit_fill(tt_ctx* c, tt_tensor* t, const int64_t* idx, float value) {
  clear_error();
  if (!c || !t) return fail(TT_ERR_ARG, "tt_submit_fill: null");
  if (int rc = check_idx(t, idx)) return rc;
  int64_t l = t->lin(idx);
  int64_t n = t->tile_elems(l);
  return c->submit("fill", {tt::W(t, l)}, [=](hipStream_t s, void*) {
    return tile_fill(s, n, (float*)t->dev(l), value);
  });
}

int tt_ctx_wait_stream(tt_ctx* c, void* stream) {
  clear_error();
  if (!c) return fail(TT_ERR_ARG, "tt_ctx_wait_stream: null");
  if (c->capturing) return fail(TT_ERR_STATE, "tt_ctx_wait_stream: a graph is being captured");
  if (c->dryrun) return TT_OK;
  // tasks still held in the window launch later, so they wait too
  if (int rc = c->ext_events_init()) return rc;
  TT_HIP_TRY(hipEventRecord(c->ext_events[0], as_stream(stream)));
  for (auto s : c->streams) TT_HIP_TRY(hipStreamWaitEvent(s, c->ext_events[0], 0));
  return TT_OK;
}

int tt_ctx_join_stream(tt_ctx* c, void* stream) {
  clear_error();
  if (!c) return fail(TT_ERR_ARG, "tt_ctx_join_stream: null");
  if (c->capturing) return fail(TT_ERR_STATE, "tt_ctx_join_stream: a graph is being captured");
  if (c->dryrun) return c->flush();
  if (int rc = c->flush()) return rc;
  if (int rc = c->ext_events_init()) return rc;
  std::vector<hipStream_t> all(c->streams);
  all.push_back(c->copy_stream);
  all.push_back(c->d2h_stream);
  for (size_t i = 0; i < all.size(); ++i) {
    TT_HIP_TRY(hipEventRecord(c->ext_events[1 + i], all[i]));
    TT_HIP_TRY(hipStreamWaitEvent(as_stream(stream), c->ext_events[1 + i], 0));
  }
  return TT_OK;
}

int tt_wait(tt_ctx* c) {
  clear_error();
  if (!c) return fail(TT_ERR_ARG, "tt_wait: null");
  return c->wait_all();
}

int tt_dump_dag(tt_ctx* c, const char* path) {
  clear_error();
  if (!c || !path) return fail(TT_ERR_ARG, "tt_dump_dag: null");
  if (int rc = c->flush()) return rc;
  std::ofstream f(path);
  if (!f) return fail(TT_ERR_ARG, "tt_dump_dag: cannot open %s", path);
  for (auto& r : c->records) {
    f << "{\"id\":" << r.id << ",\"label\":\"" << r.label << "\",\"stream\":" << r.stream
      << ",\"cost\":" << r.cost << ",\"deps\":[";
    for (size_t i = 0; i < r.deps.size(); ++i) f << (i ? "," : "") << r.deps[i];
    f << "],\"acc\":[";
    for (size_t i = 0; i < r.acc.size(); ++i)
      f << (i ? "," : "") << "[" << r.acc[i].first << "," << r.acc[i].second.first << ","
        << r.acc[i].second.second << "]";
    f << "]}\n";
  }
  return TT_OK;
}

int tt_get_stats(tt_ctx* c, tt_stats* out) {
  if (!c || !out) return fail(TT_ERR_ARG, "tt_get_stats: null");
  *out = c->stats;
  return TT_OK;
}

int tt_reset_stats(tt_ctx* c) {
  if (!c) return fail(TT_ERR_ARG, "tt_reset_stats: null");
  c->stats = tt_stats{};
  c->records.clear();
  return TT_OK;
}

}  // extern "C"

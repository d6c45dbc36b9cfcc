// Disk tier: record file and the read-ahead thread that feeds the copies.
#include "disk.h"

#include <fcntl.h>
#include <unistd.h>

#include <algorithm>
#include <cerrno>
#include <chrono>
#include <cstring>
#include <thread>
#include <vector>

namespace {

// preads per record, run concurrently.  One sequential read of the record is
// the fastest on the virtual disks measured (6.4 GB/s; 2 parts 5.6, 4 parts
// 4.8, 8 parts 3.5, 16 parts 2.4).
constexpr int kReadParts = 1;

int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// pread / pwrite of exactly n bytes (they may return short counts).
int full_pread(int fd, uint8_t* p, int64_t n, int64_t off) {
  while (n > 0) {
    const ssize_t r = ::pread(fd, p, (size_t)n, (off_t)off);
    if (r < 0) {
      if (errno == EINTR) continue;
      return -errno;
    }
    if (r == 0) return -EIO;
    p += r; off += r; n -= r;
  }
  return 0;
}

int full_pwrite(int fd, const uint8_t* p, int64_t n, int64_t off) {
  while (n > 0) {
    const ssize_t r = ::pwrite(fd, p, (size_t)n, (off_t)off);
    if (r < 0) {
      if (errno == EINTR) continue;
      return -errno;
    }
    p += r; off += r; n -= r;
  }
  return 0;
}

double ms_since(std::chrono::steady_clock::time_point t0) {
  return std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
}

}  // namespace

// ---------------------------------------------------------------- DiskFile
int DiskFile::open(const std::string& path, int64_t record_bytes, int n, std::string* why) {
  close_and_unlink();
  bytes_ = record_bytes;
  padded_ = round_up(record_bytes, kDiskAlign);
  n_ = n;
  fd_ = ::open(path.c_str(), O_RDWR | O_CREAT | O_TRUNC | O_CLOEXEC, 0600);
  if (fd_ < 0) {
    if (why) *why = "cannot create " + path + ": " + std::strerror(errno);
    return -1;
  }
  path_ = path;
  if (::ftruncate(fd_, (off_t)(padded_ * n)) != 0) {
    if (why) *why = "cannot size " + path + ": " + std::strerror(errno);
    close_and_unlink();
    return -1;
  }
  return 0;
}

int DiskFile::write(int idx, const uint8_t* rec) const {
  return full_pwrite(fd_, rec, bytes_, (int64_t)idx * padded_);
}

int DiskFile::flush_and_drop() const {
  if (::fdatasync(fd_) != 0) return -errno;
  const int rc = ::posix_fadvise(fd_, 0, (off_t)(padded_ * n_), POSIX_FADV_DONTNEED);
  return rc ? -rc : 0;
}

int DiskFile::read_from_device(int idx, uint8_t* buf, int parts) const {
  const int64_t off = (int64_t)idx * padded_;
  parts = std::max(1, std::min<int>(parts, (int)(bytes_ / (1 << 20)) + 1));
  std::vector<int> rc(parts, 0);
  std::vector<std::thread> th;
  for (int i = 0; i < parts; ++i) {
    const int64_t a = round_up(bytes_ * i / parts, kDiskAlign), b = i + 1 == parts ? bytes_ : round_up(bytes_ * (i + 1) / parts, kDiskAlign);
    if (b <= a) continue;
    th.emplace_back([&, i, a, b] { rc[i] = full_pread(fd_, buf + a, b - a, off + a); });
  }
  for (auto& x : th) x.join();
  for (int r : rc)
    if (r) return r;
  const int fr = ::posix_fadvise(fd_, (off_t)off, (off_t)padded_, POSIX_FADV_DONTNEED);
  return fr ? -fr : 0;
}

int DiskFile::read_any(int idx, uint8_t* buf) const {
  return full_pread(fd_, buf, bytes_, (int64_t)idx * padded_);
}

void DiskFile::close_and_unlink() {
  if (fd_ >= 0) ::close(fd_);
  if (!path_.empty()) ::unlink(path_.c_str());
  fd_ = -1;
  path_.clear();
}

// ---------------------------------------------------------------- DiskReader
int DiskReader::init(const DiskFile* f, int first, int n_layers, int nbuf, std::string* why) {
  f_ = f;
  first_ = first;
  n_layers_ = n_layers;
  const int fr = f->flush_and_drop();
  if (fr) {
    if (why) *why = std::string("disk tier flush failed: ") + std::strerror(-fr);
    return -1;
  }
  bufs_.resize(nbuf);
  for (auto& b : bufs_) {
    if (hipHostMalloc(reinterpret_cast<void**>(&b.p), (size_t)f->padded(), hipHostMallocDefault) != hipSuccess ||
        !b.p) {
      if (why) *why = "hipHostMalloc of a disk staging buffer failed";
      return -1;
    }
    if (hipEventCreateWithFlags(&b.copied, hipEventDisableTiming) != hipSuccess) {
      if (why) *why = "hipEventCreate failed";
      return -1;
    }
  }
  th_ = std::thread(&DiskReader::run, this);
  return 0;
}

DiskReader::~DiskReader() {
  {
    std::lock_guard<std::mutex> lk(mu_);
    stop_ = true;
  }
  cv_.notify_all();
  if (th_.joinable()) th_.join();
  for (auto& b : bufs_) {
    if (b.copied) {
      (void)hipEventSynchronize(b.copied);
      (void)hipEventDestroy(b.copied);
    }
    if (b.p) (void)hipHostFree(b.p);
  }
}

// A buffer to read `layer` into: a free one, else one holding a read-ahead
// that is ready but not taken.  With may_wait, blocks until one exists.
int DiskReader::claim(int layer, bool may_wait, std::unique_lock<std::mutex>& lk) {
  for (;;) {
    for (int i = 0; i < (int)bufs_.size(); ++i)
      if (bufs_[i].state == FREE) return i;
    for (int i = 0; i < (int)bufs_.size(); ++i)
      if (bufs_[i].state == READY && bufs_[i].layer != layer) return i;
    if (!may_wait) return -1;
    cv_.wait(lk);
  }
}

const uint8_t* DiskReader::take(int layer, int dir, int* buf) {
  const auto t0 = std::chrono::steady_clock::now();
  std::unique_lock<std::mutex> lk(mu_);
  int b = -1;
  for (int i = 0; i < (int)bufs_.size(); ++i)
    if (bufs_[i].layer == layer && (bufs_[i].state == QUEUED || bufs_[i].state == READING || bufs_[i].state == READY))
      b = i;
  if (b < 0) {
    b = claim(layer, true, lk);
    bufs_[b].layer = layer;
    bufs_[b].state = QUEUED;
    jobs_.push_back(b);
    cv_.notify_all();
  }
  cv_.wait(lk, [&] { return bufs_[b].state == READY; });
  st_.wait_ms += ms_since(t0);
  if (bufs_[b].rc) {
    err_ = std::string("disk tier read failed: ") + std::strerror(-bufs_[b].rc);
    bufs_[b].state = FREE;
    bufs_[b].layer = -1;
    return nullptr;
  }
  bufs_[b].state = TAKEN;
  // Read ahead: the next disk layer in the sweep's direction, into a free buffer.
  const int next = layer + (dir >= 0 ? 1 : -1);
  if (next >= first_ && next < n_layers_) {
    bool held = false;
    for (auto& x : bufs_)
      if (x.layer == next && x.state != FREE) held = true;
    if (!held) {
      int nb = -1;
      for (int i = 0; i < (int)bufs_.size(); ++i)
        if (bufs_[i].state == FREE) { nb = i; break; }
      if (nb >= 0) {
        bufs_[nb].layer = next;
        bufs_[nb].state = QUEUED;
        jobs_.push_back(nb);
        cv_.notify_all();
      }
    }
  }
  *buf = b;
  return bufs_[b].p;
}

int DiskReader::after_copy(int b, hipStream_t stream) {
  if (hipEventRecord(bufs_[b].copied, stream) != hipSuccess) return -1;
  std::lock_guard<std::mutex> lk(mu_);
  bufs_[b].copy_pending = true;
  bufs_[b].state = FREE;
  bufs_[b].layer = -1;
  cv_.notify_all();
  return 0;
}

void DiskReader::run() {
  for (;;) {
    int b;
    bool pending;
    int layer;
    {
      std::unique_lock<std::mutex> lk(mu_);
      cv_.wait(lk, [&] { return stop_ || !jobs_.empty(); });
      if (stop_) return;
      b = jobs_.front();
      jobs_.pop_front();
      bufs_[b].state = READING;
      pending = bufs_[b].copy_pending;
      layer = bufs_[b].layer;
    }
    // The buffer's previous record must have left for the device.
    if (pending) (void)hipEventSynchronize(bufs_[b].copied);
    const auto t0 = std::chrono::steady_clock::now();
    const int rc = f_->read_from_device(layer - first_, bufs_[b].p, kReadParts);
    const double ms = ms_since(t0);
    {
      std::lock_guard<std::mutex> lk(mu_);
      bufs_[b].copy_pending = false;
      bufs_[b].rc = rc;
      bufs_[b].state = READY;
      st_.reads += 1;
      st_.bytes += f_->record_bytes();
      st_.read_ms += ms;
    }
    cv_.notify_all();
  }
}

DiskReader::Stats DiskReader::stats() {
  std::lock_guard<std::mutex> lk(mu_);
  return st_;
}

void DiskReader::reset_stats() {
  std::lock_guard<std::mutex> lk(mu_);
  st_ = Stats{};
}
